// Weight-streaming projections for few activation rows.
//
// Y[m, n] = sum_k X[m, k] * W[n, k] where the weights dominate the bytes, so
// both kernels are organised around reading W exactly once from HBM with
// 16-byte non-temporal loads and enough of them in flight per CU:
//
// gemv_lds_kernel (M <= 8 per slice, and every fp32 model):
//   the activation slice is staged once per workgroup in LDS; each wave owns R
//   consecutive output rows, every lane streams 16-byte pieces of those rows
//   (two k-steps in flight) and multiplies them with the matching LDS piece of
//   each activation row (v_dot2_f32_bf16 for bf16).  The R*MT per-lane partial
//   sums are folded across the wave with a reduce-scatter, so every lane ends
//   with one finished dot product and applies the epilogue to it.
//
// mfma_skinny_kernel (bf16, 8 < M <= 16 per slice):
//   at 14-16 rows the VALU would be near saturation at full HBM rate, so the
//   products run on v_mfma_f32_16x16x32_bf16: the activation rows are the A
//   operand (one 16-byte piece per lane per k-step, read through the caches)
//   and 16 weight rows are the B operand, loaded straight from HBM in the MFMA
//   lane layout.  The SK waves of a workgroup split K, their partial tiles are
//   summed through LDS and wave 0 applies the epilogue.
//
// Epilogues: plain store, residual add, SiLU(gate)*up of paired gate/up rows,
// and the LM-head argmax, which keeps a running best/runner-up per activation
// row and writes one candidate per workgroup for a final merge.
#include "common.h"

namespace pe {
namespace {

// ------------------------------------------------------------------ VALU / LDS
template <typename TW, int MT, int R, Epi EPI>
__global__ __launch_bounds__(256) void gemv_lds_kernel(GemvArgs a) {
  constexpr int VE = Elem<TW>::kVec;
  constexpr int NV = R * MT;
  constexpr int SH = 6 - Log2<NV>::value;
  constexpr int RG = (EPI == Epi::SiluMul) ? R / 2 : R;  // output rows per group
  extern __shared__ u32x4 xs[];                            // [MT][K / VE]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K;
  const int KV = K / VE;
  const int m0 = blockIdx.y * MT;
  const int mcount = min(MT, a.M - m0);
  {
    const char* xb = static_cast<const char*>(a.x) + static_cast<int64_t>(m0) * K * sizeof(TW);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int v = threadIdx.x; v < MT * KV; v += blockDim.x) {
      const int m = v / KV;
      xs[v] = m < mcount ? load16(xb + static_cast<int64_t>(v) * 16) : zero;
    }
    __syncthreads();
  }
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
    for (int j = lane; j < KV; j += 128) {
      const bool two = j + 64 < KV;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      u32x4 w0[R], w1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w0[r] = load16_stream(wp[r] + j * VE);
#pragma unroll
      for (int r = 0; r < R; ++r) w1[r] = two ? load16_stream(wp[r] + (j + 64) * VE) : zero;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 x0 = xs[m * KV + j];
        const u32x4 x1 = two ? xs[m * KV + j + 64] : zero;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r * MT + m] = dot16<TW>(w0[r], x0, acc[r * MT + m]);
          acc[r * MT + m] = dot16<TW>(w1[r], x1, acc[r * MT + m]);
        }
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
        static_cast<TW*>(a.y_op)[static_cast<int64_t>(m0 + my_m) * a.ldy + n] = Elem<TW>::from_f32(s * up);
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

// ------------------------------------------------------------------ MFMA skinny
template <int SK, int U, Epi EPI>
__global__ __launch_bounds__(64 * SK) void mfma_skinny_kernel(GemvArgs a) {
  constexpr int NB = EPI == Epi::SiluMul ? 2 : 1;  // B tiles per output tile (gate, up)
  __shared__ f32x4 red[SK][NB][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K;
  const int KS = K / 32;
  const int per = (KS + SK - 1) / SK;
  const int ks0 = min(KS, wave * per);
  const int ks1 = min(KS, ks0 + per);
  const int m0 = blockIdx.y * 16;
  const int mrow = m0 + (lane & 15);
  const bool xvalid = mrow < a.M;
  const char* xp = static_cast<const char*>(a.x) +
                   (static_cast<int64_t>(min(mrow, a.M - 1)) * K + (lane >> 4) * 8) * 2;
  const int T = (a.Nout + 15) / 16;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  Top2 best[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) best[q] = top2_empty();

  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    const int n0 = t * 16;
    const int nrow = min(n0 + (lane & 15), a.Nout - 1);
    const bf16_t* wp[NB];
    if constexpr (EPI == Epi::SiluMul) {
      wp[0] = static_cast<const bf16_t*>(a.w_a) + static_cast<int64_t>(nrow) * K + (lane >> 4) * 8;
      wp[NB - 1] = static_cast<const bf16_t*>(a.w_b) + static_cast<int64_t>(nrow) * K + (lane >> 4) * 8;
    } else {
      const bf16_t* base;
      int rr;
      if (nrow < a.n_a) {
        base = static_cast<const bf16_t*>(a.w_a);
        rr = nrow;
      } else if (nrow < a.n_a + a.n_b) {
        base = static_cast<const bf16_t*>(a.w_b);
        rr = nrow - a.n_a;
      } else {
        base = static_cast<const bf16_t*>(a.w_c);
        rr = nrow - a.n_a - a.n_b;
      }
      wp[0] = base + static_cast<int64_t>(rr) * K + (lane >> 4) * 8;
    }
    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = ks0; s < ks1; s += U) {
      u32x4 av[U], bv[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = s + u < ks1;
#pragma unroll
        for (int b = 0; b < NB; ++b) bv[u][b] = ok ? load16_stream(wp[b] + (s + u) * 32) : zero;
        av[u] = (ok && xvalid) ? load16(xp + (s + u) * 64) : zero;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                           __builtin_bit_cast(bf16x8, bv[u][b]), acc[b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
    if (wave == 0) {
      f32x4 sum[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        sum[b] = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < SK; ++w) sum[b] += red[w][b][lane];
      }
      const int n = n0 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + 4 * (lane >> 4) + q;
        if (m >= a.M || n >= a.Nout) continue;
        const float v = sum[0][q];
        if constexpr (EPI == Epi::Store) {
          a.y[static_cast<int64_t>(m) * a.ldy + n] = v;
        } else if constexpr (EPI == Epi::AddTo) {
          a.y[static_cast<int64_t>(m) * a.ldy + n] += v;
        } else if constexpr (EPI == Epi::SiluMul) {
          const float s = v / (1.f + expf(-v));
          static_cast<bf16_t*>(a.y_op)[static_cast<int64_t>(m) * a.ldy + n] = f32_to_bf16(s * sum[NB - 1][q]);
        } else {
          if (a.logits) a.logits[static_cast<int64_t>(m) * a.Nout + n] = v;
          top2_push(best[q], v, n);
        }
      }
    }
    __syncthreads();
  }

  if constexpr (EPI == Epi::Argmax) {
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {
          Top2 o;
          o.v1 = __shfl_xor(best[q].v1, off, 64);
          o.i1 = __shfl_xor(best[q].i1, off, 64);
          o.v2 = __shfl_xor(best[q].v2, off, 64);
          o.pad = 0;
          best[q] = top2_merge(best[q], o);
        }
        const int m = m0 + 4 * (lane >> 4) + q;
        if ((lane & 15) == 0 && m < a.M) a.partials[static_cast<int64_t>(m) * gridDim.x + blockIdx.x] = best[q];
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
// Smallest activation-row tile that covers M (one pass over the weights),
// 16-row slices beyond that.
int gemv_m_tile(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

bool use_mfma(int M, int K, DType dt) { return dt == DType::BF16 && M > 8 && K % 32 == 0; }

int skinny_sk(int K) { return K >= 4096 ? 8 : 4; }

template <typename TW, int MT, int R, Epi EPI>
hipError_t launch_lds(GemvArgs& a, dim3 grid, hipStream_t s) {
  const size_t lds = static_cast<size_t>(MT) * a.K * sizeof(TW);
  static bool raised = false;
  if (lds > 64 * 1024 && !raised) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_lds_kernel<TW, MT, R, EPI>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return hipErrorInvalidValue;
    raised = true;
  }
  hipLaunchKernelGGL((gemv_lds_kernel<TW, MT, R, EPI>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <typename TW, Epi EPI>
hipError_t launch_typed(GemvArgs& a, int num_cus, hipStream_t s) {
  if (use_mfma(a.M, a.K, sizeof(TW) == 2 ? DType::BF16 : DType::F32)) {
    if constexpr (sizeof(TW) == 2) {
      const int T = (a.Nout + 15) / 16;
      int gx = T < num_cus * 4 ? T : num_cus * 4;
      a.grid_x = gx;
      dim3 grid(gx, (a.M + 15) / 16);
      if (skinny_sk(a.K) == 8)
        hipLaunchKernelGGL((mfma_skinny_kernel<8, 8, EPI>), grid, dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((mfma_skinny_kernel<4, 8, EPI>), grid, dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  const int m_tile = gemv_m_tile(a.M);
  const int R = m_tile >= 16 ? 4 : m_tile >= 8 ? 8 : 16;  // R * MT <= 64
  const int rg = EPI == Epi::SiluMul ? R / 2 : R;
  const int groups = (a.Nout + rg - 1) / rg;
  int gx = (groups + 3) / 4;
  if (gx > num_cus) gx = num_cus;
  if (gx < 1) gx = 1;
  a.grid_x = gx;
  dim3 grid(gx, (a.M + m_tile - 1) / m_tile);
  switch (m_tile) {
    case 16: return launch_lds<TW, 16, 4, EPI>(a, grid, s);
    case 8: return launch_lds<TW, 8, 8, EPI>(a, grid, s);
    case 4: return launch_lds<TW, 4, 16, EPI>(a, grid, s);
    case 2: return launch_lds<TW, 2, 16, EPI>(a, grid, s);
    default: return launch_lds<TW, 1, 16, EPI>(a, grid, s);
  }
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

int gemv_grid_x(int M, int Nout, Epi epi, DType dt, int num_cus, int K) {
  if (use_mfma(M, K, dt)) {
    const int T = (Nout + 15) / 16;
    return T < num_cus * 4 ? T : num_cus * 4;
  }
  const int m_tile = gemv_m_tile(M);
  const int R = m_tile >= 16 ? 4 : m_tile >= 8 ? 8 : 16;
  const int rg = epi == Epi::SiluMul ? R / 2 : R;
  int gx = ((Nout + rg - 1) / rg + 3) / 4;
  if (gx > num_cus) gx = num_cus;
  return gx < 1 ? 1 : gx;
}

size_t gemv_lds_bytes(int M, int K, DType dt) {
  if (use_mfma(M, K, dt)) return 0;
  return static_cast<size_t>(gemv_m_tile(M)) * K * elem_bytes(dt);
}

hipError_t launch_gemv(GemvArgs& a, Epi epi, DType dt, int num_cus, hipStream_t s) {
  if (dt == DType::F32) return launch_dtype<float>(a, epi, num_cus, s);
  return launch_dtype<bf16_t>(a, epi, num_cus, s);
}

}  // namespace pe
