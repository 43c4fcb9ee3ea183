// Dense projections for decode-sized batches (T <= 64): split-K streaming GEMV.
//
// At decode the two latent projections and the router read 128 MB of weights
// for 16 tokens, so they are bound by HBM like the experts. Each wave streams
// 32 weight rows over one K slice: every load instruction covers 4 rows x 256
// contiguous bytes (read-once cache policy), staged through a wave-private
// XOR-swizzled LDS tile into bf16 MFMA 16x16x32 fragments. K is split across
// waves so that a few hundred blocks cover the chip; partial sums go to fp32
// planes [slice][token][row] and are summed in a fixed slice order by the
// consumer (the route kernel for the latent row and the logits, finish_up for
// the output), so results stay run-to-run identical.
//
// fp32 router weights are split exactly into three bf16 planes (truncation:
// w = hi + mid + lo), so each partial is a sum of exact bf16 products in fp32.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Steps of a slice run in blocks of kRun straight-line steps through a ring of three register
// stages. Every step issues its loads (a step past the slice reads zeros from a zero-size
// resource), so no load sits under a branch and the compiler's waits count exactly the loads
// in flight; a branch or a loop back edge between a load and its use makes it wait for all.
constexpr int kRun = 8;
constexpr int kStepBytes = 256;  // bytes of each weight row per step
constexpr int kGemvCus = 256;    // MI355X compute units

template <int MT, bool F32>
__device__ __forceinline__ void gemv_body(const GemvArgs& args, const GemvSeg& sg, int slice, int row0, int wave,
                                          uint8_t* lds) {
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, q = lane >> 4;
  constexpr int kEs = F32 ? 4 : 2;                    // bytes per weight
  constexpr int kKs = F32 ? 2 : 4;                    // MFMA k-steps (32 K each) per 256-byte step
  const int K = args.K;
  const uint32_t rowb = (uint32_t)K * kEs;            // bytes per weight row
  const int nsteps = (int)(rowb / kStepBytes);        // 256 bytes of every row per step
  const int per = (nsteps + sg.splits - 1) / sg.splits;
  const int s0 = slice * per, s1 = min(nsteps, s0 + per);
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(sg.W, (uint32_t)sg.N * rowb);
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(args.A, 0x7fffffffu);
  const __amdgpu_buffer_rsrc_t none = make_rsrc(sg.W, 0u);

  // load l covers rows 4l .. 4l+3 of the wave's 32, 16 lanes x 16 bytes per row; LDS row j holds
  // its 16 chunks XOR-swizzled by j, so the 16-byte writes and the fragment reads (16 rows, one
  // chunk each) are bank-conflict free
  uint32_t goff[8], wlds[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    const int j = 4 * l + (lane >> 4), c = lane & 15;
    const int row = min(row0 + j, sg.N - 1);  // rows past N are never stored
    goff[l] = (uint32_t)row * rowb + c * 16;
    wlds[l] = j * kStepBytes + ((c ^ (j & 15)) * 16);
  }
  auto frag = [&](int t, int c) -> uint32_t {
    const int j = 16 * t + nl;
    return j * kStepBytes + ((c ^ nl) * 16);
  };
  uint32_t aoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + nl;
    aoff[mt] = m < args.M ? ((uint32_t)m * (uint32_t)args.lda + q * 8) * 2 : 0x80000000u;
  }

  f32x4_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    u32x4_t w[8];
    u32x4_t x[MT][kKs];
  };
  auto issue = [&](Stage& st, int s) {  // step s, or zeros past the slice
    const bool on = s < s1;
    const uint32_t kb = (uint32_t)s * kStepBytes;
#pragma unroll
    for (int l = 0; l < 8; ++l) st.w[l] = buf_load16_nt(on ? w_rs : none, goff[l] + kb);
    const uint32_t kelem = kb / kEs;  // first K index of the step
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < kKs; ++h)
        st.x[mt][h] = buf_load16(on ? a_rs : none,
                                 aoff[mt] == 0x80000000u ? aoff[mt] : aoff[mt] + (kelem + h * 32) * 2);
  };
  auto consume = [&](const Stage& st) {
#pragma unroll
    for (int l = 0; l < 8; ++l) *(u32x4_t*)(lds + wlds[l]) = st.w[l];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!F32) {
#pragma unroll
        for (int h = 0; h < kKs; ++h) {
          const u32x4_t wf = *(const u32x4_t*)(lds + frag(t, 4 * h + q));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[mt][h]), as_bf16x8(wf), acc[mt][t], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int h = 0; h < kKs; ++h) {
          const u32x4_t w0 = *(const u32x4_t*)(lds + frag(t, 8 * h + 2 * q));
          const u32x4_t w1 = *(const u32x4_t*)(lds + frag(t, 8 * h + 2 * q + 1));
          uint32_t h4[4], m4[4], l4[4];
          split3x2(__uint_as_float(w0[0]), __uint_as_float(w0[1]), h4[0], m4[0], l4[0]);
          split3x2(__uint_as_float(w0[2]), __uint_as_float(w0[3]), h4[1], m4[1], l4[1]);
          split3x2(__uint_as_float(w1[0]), __uint_as_float(w1[1]), h4[2], m4[2], l4[2]);
          split3x2(__uint_as_float(w1[2]), __uint_as_float(w1[3]), h4[3], m4[3], l4[3]);
          const u32x4_t hi = {h4[0], h4[1], h4[2], h4[3]};
          const u32x4_t mi = {m4[0], m4[1], m4[2], m4[3]};
          const u32x4_t lo = {l4[0], l4[1], l4[2], l4[3]};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[mt][h]), as_bf16x8(hi), acc[mt][t], 0, 0, 0);
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[mt][h]), as_bf16x8(mi), acc[mt][t], 0, 0, 0);
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[mt][h]), as_bf16x8(lo), acc[mt][t], 0, 0, 0);
          }
        }
      }
    }
  };

  // the fences keep each step's loads ahead of the previous step's compute (the scheduler
  // would otherwise sink them and wait for everything in flight)
  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int b = s0; b < s1; b += kRun) {
    Stage st[3];
    issue(st[0], b);
    issue(st[1], b + 1);
    fence();
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      if (i + 2 < kRun) issue(st[(i + 2) % 3], b + i + 2);
      fence();
      consume(st[i % 3]);
      fence();
    }
  }

  // partial sums of this slice: lane holds D[m = 4q + r][n = nl] of each tile
  float* part = sg.part + (size_t)slice * args.M * sg.N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = row0 + 16 * t + nl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * 16 + 4 * q + r;
        if (m < args.M && n < sg.N) part[(size_t)m * sg.N + n] = acc[mt][t][r];
      }
    }
}

// WPB waves per block, each 32 rows of one K slice. The waves share nothing (each has its own
// LDS tile and no barrier). Four-wave blocks when the launch has at most one per compute unit;
// otherwise single-wave blocks, which the dispatcher spreads evenly (with a few hundred 4-wave
// blocks of equal bytes, some units got two blocks' work and the rest one).
template <int MT, int WPB>
__global__ __launch_bounds__(64 * WPB) void dense_gemv_kernel(GemvArgs args, int blocks0, int bands0, int bands1) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[WPB][32 * kStepBytes];
  const int wave = threadIdx.x >> 6;
  const bool second = (int)blockIdx.x >= blocks0;
  const int local = second ? (int)blockIdx.x - blocks0 : (int)blockIdx.x;
  const GemvSeg& sg = args.seg[second ? 1 : 0];
  const int bands = second ? bands1 : bands0;
  const int band = local % bands, slice = local / bands;
  const int row0 = (band * WPB + wave) * 32;
  if (row0 >= sg.N) return;  // wave-uniform; no block barrier in this kernel
  // weight format uniform over the block, taken once outside the step loop
  if (sg.w_f32)
    gemv_body<MT, true>(args, sg, slice, row0, wave, lds_all[wave]);
  else
    gemv_body<MT, false>(args, sg, slice, row0, wave, lds_all[wave]);
}

__global__ __launch_bounds__(256) void finish_up_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                        const float* __restrict__ addend, uint16_t* __restrict__ y,
                                                        float* __restrict__ tap, RowScale rs) {
  const size_t total = (size_t)M * N / 4;
  const size_t plane = (size_t)M * N;
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) acc += *(const f32x4_t*)(part + s * plane + 4 * i);
    if (rs.part_sq) {  // the row's RMSNorm factor, from its column blocks' sums of squares
      const size_t m = 4 * i / N;
      float tot = 0.f;
      for (int q = 0; q < rs.nq; ++q) tot += rs.part_sq[m * rs.nq + q];
      acc *= rsqrtf(tot / (float)rs.L + rs.eps);
    }
    if (tap) *(f32x4_t*)(tap + 4 * i) = acc;
    if (addend) acc += *(const f32x4_t*)(addend + 4 * i);
    *(uint2*)(y + 4 * i) = uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
}

template <int WPB>
hipError_t launch_kind(const GemvArgs& a, int blocks0, int bands0, int bands1, int total, hipStream_t s) {
  const int mt = (a.M + 15) / 16;
  if (mt <= 1)
    hipLaunchKernelGGL((dense_gemv_kernel<1, WPB>), dim3(total), dim3(64 * WPB), 0, s, a, blocks0, bands0, bands1);
  else if (mt <= 2)
    hipLaunchKernelGGL((dense_gemv_kernel<2, WPB>), dim3(total), dim3(64 * WPB), 0, s, a, blocks0, bands0, bands1);
  else
    hipLaunchKernelGGL((dense_gemv_kernel<4, WPB>), dim3(total), dim3(64 * WPB), 0, s, a, blocks0, bands0, bands1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_gemv(const GemvArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.M > 64) return hipErrorInvalidValue;
  int bands[2] = {1, 1}, blocks[2] = {0, 0};
  for (int i = 0; i < a.nseg; ++i) {
    bands[i] = (a.seg[i].N + 127) / 128;
    blocks[i] = bands[i] * a.seg[i].splits;
  }
  if (blocks[0] + blocks[1] <= kGemvCus) return launch_kind<4>(a, blocks[0], bands[0], bands[1], blocks[0] + blocks[1], s);
  for (int i = 0; i < a.nseg; ++i) {
    bands[i] = (a.seg[i].N + 31) / 32;
    blocks[i] = bands[i] * a.seg[i].splits;
  }
  return launch_kind<1>(a, blocks[0], bands[0], bands[1], blocks[0] + blocks[1], s);
}

hipError_t launch_finish_up(const float* part, int splits, int M, int N, const float* addend, uint16_t* y, float* tap,
                            RowScale rs, hipStream_t s) {
  const size_t total = (size_t)M * N / 4;
  if (!total) return hipSuccess;
  const size_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(finish_up_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, s, part, splits,
                     M, N, addend, y, tap, rs);
  return hipGetLastError();
}

}  // namespace moe
