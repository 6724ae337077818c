// Weight-streaming skinny GEMM ("GEMV") for the drafter's projections.
//
// Y[m, n] = sum_k X[m, k] * W[n, k] with few activation rows (M <= 16 per
// launch slice).  The weights dominate the bytes, so the kernel is built
// around streaming W once from HBM at full width:
//   * each wave owns R consecutive output rows at a time; every lane loads
//     16-byte slices of those R weight rows (non-temporal, they are read once)
//     at k-vectors lane, lane+64, ... and the matching 16-byte slices of the
//     MT activation rows, which stay hot in the caches;
//   * products are accumulated in fp32 (v_dot2_f32_bf16 for bf16 weights);
//   * the R*MT per-lane partial sums are folded across the wave with a
//     reduce-scatter, so each lane ends with one finished dot product and
//     applies the epilogue to it;
//   * the grid is persistent-style (a few workgroups per CU, grid-stride over
//     row groups), and rows of M beyond MT are handled by blockIdx.y slices.
// Epilogues: plain store, residual add, SiLU(gate)*up of paired gate/up rows,
// and the LM-head argmax, which keeps a running best/runner-up per activation
// row and writes one candidate per workgroup for a final merge.
#include "common.h"

namespace pe {
namespace {

template <typename TW, int MT, int R, Epi EPI>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  constexpr int VE = Elem<TW>::kVec;
  constexpr int NV = R * MT;
  constexpr int SH = 6 - Log2<NV>::value;
  constexpr int RG = (EPI == Epi::SiluMul) ? R / 2 : R;  // output rows per group
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K;
  const int KV = K / VE;
  const int m0 = blockIdx.y * MT;
  const int mcount = min(MT, a.M - m0);
  const int64_t xrow = static_cast<int64_t>(K) * sizeof(TW);
  const char* xb = static_cast<const char*>(a.x) + m0 * xrow;
  const int G = (a.Nout + RG - 1) / RG;
  const int idx = lane >> SH;
  const int my_r = idx / MT;
  const int my_m = idx % MT;
  const bool owner = (lane & ((1 << SH) - 1)) == 0;
  Top2 best = top2_empty();

  for (int g = blockIdx.x * 4 + wave; g < G; g += gridDim.x * 4) {
    const int n0 = g * RG;
    const TW* wp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (EPI == Epi::SiluMul) {
        const int n = min(n0 + (r % RG), a.Nout - 1);
        wp[r] = static_cast<const TW*>(r < RG ? a.w_a : a.w_b) + static_cast<int64_t>(n) * K;
      } else {
        const int n = min(n0 + r, a.Nout - 1);
        if (n < a.n_a)
          wp[r] = static_cast<const TW*>(a.w_a) + static_cast<int64_t>(n) * K;
        else if (n < a.n_a + a.n_b)
          wp[r] = static_cast<const TW*>(a.w_b) + static_cast<int64_t>(n - a.n_a) * K;
        else
          wp[r] = static_cast<const TW*>(a.w_c) + static_cast<int64_t>(n - a.n_a - a.n_b) * K;
      }
    }
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
    for (int j = lane; j < KV; j += 64) {
      u32x4 w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = load16_stream(wp[r] + j * VE);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mm = m < mcount ? m : mcount - 1;
        const u32x4 x = load16(xb + mm * xrow + j * 16);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r * MT + m] = dot16<TW>(w[r], x, acc[r * MT + m]);
      }
    }
    const float val = wave_reduce_scatter<NV>(acc, lane);
    const int n = n0 + my_r;
    if constexpr (EPI == Epi::Store || EPI == Epi::AddTo) {
      if (owner && n < a.Nout && my_m < mcount) {
        float* y = a.y + static_cast<int64_t>(m0 + my_m) * a.ldy + n;
        if constexpr (EPI == Epi::Store) *y = val;
        else *y += val;
      }
    } else if constexpr (EPI == Epi::SiluMul) {
      const float up = __shfl(val, ((idx + RG * MT) << SH) & 63, 64);
      if (owner && my_r < RG && n < a.Nout && my_m < mcount) {
        const float s = val / (1.f + expf(-val));
        static_cast<TW*>(a.y_op)[static_cast<int64_t>(m0 + my_m) * a.ldy + n] =
            Elem<TW>::from_f32(s * up);
      }
    } else {  // Argmax
      if (owner && n < a.Nout && my_m < mcount) {
        if (a.logits) a.logits[static_cast<int64_t>(m0 + my_m) * a.Nout + n] = val;
        top2_push(best, val, n);
      }
    }
  }

  if constexpr (EPI == Epi::Argmax) {
    constexpr int RBIT = SH + Log2<MT>::value;  // lane bits that select the row r
#pragma unroll
    for (int off = 32; off >= (1 << RBIT) && off >= 1; off >>= 1) {
      Top2 o;
      o.v1 = __shfl_xor(best.v1, off, 64);
      o.i1 = __shfl_xor(best.i1, off, 64);
      o.v2 = __shfl_xor(best.v2, off, 64);
      o.pad = 0;
      best = top2_merge(best, o);
    }
    __shared__ Top2 red[4][MT];
    if (owner && my_r == 0) red[wave][my_m] = best;
    __syncthreads();
    if (threadIdx.x < MT && static_cast<int>(threadIdx.x) < mcount) {
      Top2 t = red[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < 4; ++w) t = top2_merge(t, red[w][threadIdx.x]);
      a.partials[static_cast<int64_t>(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = t;
    }
  }
}

template <typename TW, Epi EPI>
hipError_t launch_typed(GemvArgs& a, int num_cus, hipStream_t s) {
  const int m_tile = a.M >= 16 ? 16 : a.M >= 8 ? 8 : a.M >= 4 ? 4 : a.M >= 2 ? 2 : 1;
  // rows per wave: R * MT <= 64
  const int R = m_tile >= 16 ? 4 : m_tile >= 8 ? 8 : 16;
  const int rg = EPI == Epi::SiluMul ? R / 2 : R;
  const int groups = (a.Nout + rg - 1) / rg;
  int gx = (groups + 3) / 4;
  const int cap = num_cus * 2;
  if (gx > cap) gx = cap;
  if (gx < 1) gx = 1;
  a.grid_x = gx;
  dim3 grid(gx, (a.M + m_tile - 1) / m_tile);
  switch (m_tile) {
    case 16: hipLaunchKernelGGL((gemv_kernel<TW, 16, 4, EPI>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<TW, 8, 8, EPI>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<TW, 4, 16, EPI>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<TW, 2, 16, EPI>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<TW, 1, 16, EPI>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <typename TW>
hipError_t launch_dtype(GemvArgs& a, Epi epi, int num_cus, hipStream_t s) {
  switch (epi) {
    case Epi::Store: return launch_typed<TW, Epi::Store>(a, num_cus, s);
    case Epi::AddTo: return launch_typed<TW, Epi::AddTo>(a, num_cus, s);
    case Epi::SiluMul: return launch_typed<TW, Epi::SiluMul>(a, num_cus, s);
    default: return launch_typed<TW, Epi::Argmax>(a, num_cus, s);
  }
}

}  // namespace

int gemv_grid_x(int M, int Nout, Epi epi, DType, int num_cus) {
  const int m_tile = M >= 16 ? 16 : M >= 8 ? 8 : M >= 4 ? 4 : M >= 2 ? 2 : 1;
  const int R = m_tile >= 16 ? 4 : m_tile >= 8 ? 8 : 16;
  const int rg = epi == Epi::SiluMul ? R / 2 : R;
  int gx = ((Nout + rg - 1) / rg + 3) / 4;
  if (gx > num_cus * 2) gx = num_cus * 2;
  return gx < 1 ? 1 : gx;
}

hipError_t launch_gemv(GemvArgs& a, Epi epi, DType dt, int num_cus, hipStream_t s) {
  if (dt == DType::F32) return launch_dtype<float>(a, epi, num_cus, s);
  return launch_dtype<bf16_t>(a, epi, num_cus, s);
}

}  // namespace pe
