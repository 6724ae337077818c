// Weight-streaming projections for few activation rows.
//
// Y[m, n] = sum_k X[m, k] * W[n, k] where the weights dominate the bytes, so
// both kernels are organised around reading W exactly once from HBM with
// 16-byte loads and enough of them in flight per CU:
//
// gemv_lds_kernel (every fp32 model, and the bf16 LM head over M <= 8 rows):
//   the activation slice is staged once per workgroup in LDS; each wave owns R
//   consecutive output rows, every lane streams 16-byte pieces of those rows
//   (two k-steps in flight, non-temporal) and multiplies them with the matching
//   LDS piece of each activation row (v_dot2_f32_bf16 for bf16).  The R*MT
//   per-lane partial sums are folded across the wave with a reduce-scatter, so
//   every lane ends with one finished dot product and applies the epilogue.
//
// mfma_skinny_kernel (bf16, M <= 16; the LM head from 9 rows):
//   at 14-16 rows the VALU would be near saturation at full HBM rate, so the
//   products run on v_mfma_f32_16x16x32_bf16 (fewer rows only pad the
//   fragment, and the packed weights stream better than the LDS kernel's
//   row-major ones for the layer projections): the activation rows are the A
//   operand (one 16-byte piece per lane per k-step) and 16 weight rows are the
//   B operand.  The weights come from a packed copy in MFMA fragment order
//   (each wave load one contiguous KiB) or, for the LM head and unpacked
//   models, straight from row-major W.  A workgroup owns 1, 2 or 4 column
//   tiles (one A fragment feeds all of them) and one of `splits` ranges of K;
//   its waves split that range again and meet in LDS.
//
// The activation operand can be formed on the fly (AMode): the fc input
// concatenation [emb(id) ; h], or RMSNorm of fp32 residual rows whose sums of
// squares arrive as per-tile partials from the kernel that produced them
// (Store/AddTo epilogues emit them) for the LM head.  Epilogues: store,
// residual add (or split partials that the next RMSNorm adds up),
// SiLU(gate)*up, LM-head argmax candidates, and q/k/v with RoPE and the paged
// KV write.
#include "common.h"

namespace pe {
namespace {

// 1 / sqrt(sum_t ss[t * ld + r] / K + eps), reduced over `lanes` lanes of a wave
__device__ __forceinline__ float inv_rms_of(const GemvArgs& a, int r, int lane_in, int lanes) {
  float s = 0.f;
  for (int t = lane_in; t < a.ss_tiles; t += lanes) s += a.ss[static_cast<int64_t>(t) * a.ss_ld + r];
  for (int off = lanes / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return 1.f / sqrtf(s / static_cast<float>(a.K) + a.eps);
}

// 16 bytes of activation row m starting at element kv * VE, formed per AMode.
template <typename TW, AMode MODE>
__device__ __forceinline__ u32x4 load_a16(const GemvArgs& a, int m, int kv, float inv) {
  constexpr int VE = Elem<TW>::kVec;
  if constexpr (MODE == AMode::Plain) {
    return load16(static_cast<const TW*>(a.x) + static_cast<int64_t>(m) * a.K + kv * VE);
  } else if constexpr (MODE == AMode::Gather) {
    const int half = a.K / 2;
    const int k = kv * VE;
    if (k < half) return load16(static_cast<const TW*>(a.embed) + static_cast<int64_t>(a.ids[m]) * half + k);
    return load16(static_cast<const TW*>(a.x2) + static_cast<int64_t>(m) * half + (k - half));
  } else {
    const int r = a.rows ? a.rows[m] : m;
    const float* xr = a.xf + static_cast<int64_t>(r) * a.K + kv * VE;
    const u32x4 g = load16(static_cast<const TW*>(a.gain) + kv * VE);
    u32x4 out;
    if constexpr (VE == 8) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(xr);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(xr + 4);
      const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t gw = g[e];
        const float ga = bf16_to_f32(static_cast<bf16_t>(gw & 0xffffu));
        const float gb = bf16_to_f32(static_cast<bf16_t>(gw >> 16));
        out[e] = static_cast<uint32_t>(f32_to_bf16(xs[2 * e] * inv * ga)) |
                 (static_cast<uint32_t>(f32_to_bf16(xs[2 * e + 1] * inv * gb)) << 16);
      }
    } else {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(xr);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t gw = g[e];
        out[e] = __float_as_uint(x0[e] * inv * __uint_as_float(gw));
      }
    }
    return out;
  }
}

// ------------------------------------------------------------------ VALU / LDS
template <typename TW, int MT, int R, Epi EPI, AMode MODE, int JS = 2>
__global__ __launch_bounds__(256) void gemv_lds_kernel(GemvArgs a) {
  constexpr int VE = Elem<TW>::kVec;
  constexpr int NV = R * MT;
  constexpr int SH = 6 - Log2<NV>::value;
  constexpr int RG = (EPI == Epi::SiluMul) ? R / 2 : R;  // output rows per group
  extern __shared__ u32x4 xs[];                            // [MT][K / VE]
  __shared__ float inv_s[MT];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K;
  const int KV = K / VE;
  const int m0 = blockIdx.y * MT;
  const int mcount = min(MT, a.M - m0);
  {
    if constexpr (MODE == AMode::Norm) {
      for (int m = wave; m < mcount; m += 4) {
        const int r = a.rows ? a.rows[m0 + m] : m0 + m;
        const float inv = inv_rms_of(a, r, lane, 64);
        if (lane == 0) inv_s[m] = inv;
      }
      __syncthreads();
    }
    // eight pieces per thread requested before any is stored (one at a time,
    // each LDS store would wait for its load: a round trip per piece)
    const u32x4 zero = {0u, 0u, 0u, 0u};
    constexpr int SU = 8;
    for (int v0 = threadIdx.x; v0 < MT * KV; v0 += blockDim.x * SU) {
      u32x4 piece[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int v = min(v0 + u * static_cast<int>(blockDim.x), MT * KV - 1);
        const int m = v / KV;
        piece[u] = m < mcount ? load_a16<TW, MODE>(a, m0 + m, v - m * KV, MODE == AMode::Norm ? inv_s[m] : 0.f)
                              : zero;
      }
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (v0 + u * static_cast<int>(blockDim.x) < MT * KV) xs[v0 + u * blockDim.x] = piece[u];
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
    // JS 64-lane k-steps of all R rows are requested before any is used
    for (int j = lane; j < KV; j += 64 * JS) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      u32x4 wv[JS][R];
#pragma unroll
      for (int js = 0; js < JS; ++js)
#pragma unroll
        for (int r = 0; r < R; ++r)
          wv[js][r] = (js == 0 || j + 64 * js < KV) ? load16_stream(wp[r] + (j + 64 * js) * VE) : zero;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int js = 0; js < JS; ++js) {
          const u32x4 xv = (js == 0 || j + 64 * js < KV) ? xs[m * KV + j + 64 * js] : zero;
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r * MT + m] = dot16<TW>(wv[js][r], xv, acc[r * MT + m]);
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
// Row of W feeding column c (0..15) of tile t.  For the q/k/v projection a tile
// holds 8 rotary pairs of one head: columns c and c+8 are elements j and j + d/2.
__device__ __forceinline__ int rope_tile_row(int t, int c, int d) {
  const int per_head = d / 16;
  const int head = t / per_head, p = t - head * per_head;
  return head * d + 8 * p + (c & 7) + (c >= 8 ? d / 2 : 0);
}
template <Epi EPI>
__device__ __forceinline__ int tile_row(const GemvArgs& a, int t, int c) {
  if constexpr (EPI == Epi::QkvRope) return rope_tile_row(t, c, a.rope.d);
  else return t * 16 + c;
}

// Weight-streaming MFMA projection of at most 16 activation rows.
//
// Grid (groups, splits).  Workgroup (g, z) owns the NT 16-column tiles
// [g NT, g NT + NT) (grid-stride over groups) and the z-th of `splits` equal
// ranges of k-steps (32 elements each); its SK waves divide that range again.
// Per k-step a wave loads one A fragment (activation rows, one 16-byte piece
// per lane) and NT * NB B fragments, so the activation traffic is 1 / (NT NB)
// of the weight traffic.  B fragments come either from the packed copy, where
// fragment (t, s) is one contiguous KiB and a wave's load is fully coalesced,
// or straight from row-major W (64 bytes of each of 16 rows).
//
// The steady state is branch-free.  Packed B fragments are read through a
// buffer resource per wave and tile that spans exactly the wave's fragments, so
// k-steps past the range (and tiles past the end) read zeros without touching
// memory; row-major B and the A fragments clamp such steps to the last valid
// one (A is then zeroed), and tiles past the end to the last tile (their
// columns are dropped by the epilogue).
// The SK partial tiles meet in LDS and wave n finishes tile n of the group.
// With splits > 1 (Store / AddTo only) the finished sums go to part[z] and the
// consumer adds the splits (and the residual for AddTo) in a fixed order.
template <int SK, int NT, int U, Epi EPI, AMode MODE, bool PACKED>
__global__ __launch_bounds__(64 * SK) void mfma_skinny_kernel(GemvArgs a) {
  static_assert(NT <= SK, "one finishing wave per tile");
  static_assert(EPI != Epi::Argmax || NT == 1, "argmax candidates are kept by wave 0");
  constexpr int NB = EPI == Epi::SiluMul ? 2 : 1;  // B fragments per tile (gate, up)
  constexpr int WSTEP = 32;                          // row-major: elements between k-steps of a lane's B stream
  __shared__ f32x4 red[SK][NT * NB][64];
  __shared__ float inv_s[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.K;
  const int KS = K / 32;
  const int splits = gridDim.y, z = blockIdx.y;
  const int per_z = (KS + splits - 1) / splits;
  const int kz0 = min(KS, z * per_z), kz1 = min(KS, kz0 + per_z);
  const int per = (kz1 - kz0 + SK - 1) / SK;
  const int ks0 = min(kz1, kz0 + wave * per);
  const int ks1 = min(kz1, ks0 + per);
  const int slast = max(ks0, ks1 - 1);             // clamp target (never read when ks0 == ks1)
  // (the live-row count a.m_live is not read: the one 16-row fragment always
  // holds a live row, and padding rows are computed like the others)
  const int mrow = lane & 15;
  const bool xvalid = mrow < a.M;
  const int mclamp = min(mrow, a.M - 1);
  const int j = lane >> 4;
  if constexpr (MODE == AMode::Norm) {
    for (int m = wave; m < 16; m += SK) {
      if (m < a.M) {
        const int r = a.rows ? a.rows[m] : m;
        const float inv = inv_rms_of(a, r, lane, 64);
        if (lane == 0) inv_s[m] = inv;
      }
    }
    __syncthreads();
  }
  const float inv = (MODE == AMode::Norm && xvalid) ? inv_s[lane & 15] : 0.f;
  // gathered operand [emb(id) ; h]: the token id is requested once, here, and
  // each step's piece is addressed by a select between the two row halves (a
  // per-step id load behind a branch costs a round trip per step, each
  // waiting for every load issued before it)
  const int half_k = MODE == AMode::Gather ? K / 2 : 0;
  int idm = 0;
  if constexpr (MODE == AMode::Gather) idm = a.ids[mclamp];
  const int T = (a.Nout + 15) / 16;
  const int G = (T + NT - 1) / NT;
  // q/k/v epilogue: the rejected flag and cache slot of this lane's
  // four output rows are read once, before the weights stream
  int64_t r_slot[4] = {-1, -1, -1, -1};
  bool r_live[4] = {false, false, false, false};
  if constexpr (EPI == Epi::QkvRope) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 4 * j + q;
      if (m < a.M) {
        r_live[q] = !a.rope.rejected[m];
        r_slot[q] = a.rope.slot[m];
      }
    }
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  Top2 best[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) best[q] = top2_empty();

  for (int g = blockIdx.x; g < G; g += gridDim.x) {
    const bf16_t* wp[NT][NB];
    __amdgpu_buffer_rsrc_t rs[NT][NB];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = min(g * NT + n, T - 1);
      if constexpr (PACKED) {
        // fragments (t, ks0 .. ks1) of this wave; none for tiles past the end
        const int bytes = g * NT + n < T ? (ks1 - ks0) * 1024 : 0;
        const int64_t first = (static_cast<int64_t>(t) * KS + ks0) * 512;
        rs[n][0] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(static_cast<const bf16_t*>(a.pk_a) + first), 0, bytes, kBufferDword3);
        if constexpr (NB == 2)
          rs[n][NB - 1] = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<bf16_t*>(static_cast<const bf16_t*>(a.pk_b) + first), 0, bytes, kBufferDword3);
      } else {
        const int nrow = min(tile_row<EPI>(a, t, lane & 15), a.Nout - 1);
        if constexpr (EPI == Epi::SiluMul) {
          wp[n][0] = static_cast<const bf16_t*>(a.w_a) + static_cast<int64_t>(nrow) * K + j * 8;
          wp[n][NB - 1] = static_cast<const bf16_t*>(a.w_b) + static_cast<int64_t>(nrow) * K + j * 8;
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
          wp[n][0] = base + static_cast<int64_t>(rr) * K + j * 8;
        }
      }
    }
    // q/k/v epilogue: the rotary cos/sin of the tile this wave finishes, read
    // before the weights stream rather than after it (clamped rows and tiles
    // read valid entries that the epilogue does not use)
    float2 rot[4];
    if constexpr (EPI == Epi::QkvRope) {
      const int d = a.rope.d;
      const int n = tile_row<EPI>(a, min(g * NT + min(wave, NT - 1), T - 1), lane & 15);
      const int jj = (n % d) % (d / 2);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rot[q] = a.rope.table[static_cast<int64_t>(min(4 * j + q, a.M - 1)) * (d / 2) + jj];
    }
    f32x4 acc[NT][NB];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[n][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = ks0; s < ks1; s += U) {
      // Issue order: the A fragments (cache hits) first, then the B fragments
      // step by step, all before the first product; the barrier keeps the
      // scheduler from sinking loads below products, so the products of step
      // u wait only for the loads of steps <= u.  A gathered operand goes
      // last instead: its addresses wait for the token ids, and the weight
      // stream should not wait with them.
      u32x4 av[U], bv[U][NT][NB];
      auto load_a = [&]() __attribute__((always_inline)) {
        if constexpr (MODE == AMode::Gather) {
          // the id is first needed here, after the weight loads: the empty asm
          // keeps the row address from being formed (and the id waited for)
          // ahead of them
          int id = idm;
          asm volatile("" : "+v"(id));
          const bf16_t* erow = static_cast<const bf16_t*>(a.embed) + static_cast<int64_t>(id) * half_k;
          const bf16_t* hrow = static_cast<const bf16_t*>(a.x2) + static_cast<int64_t>(mclamp) * half_k - half_k;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int k = (4 * min(s + u, slast) + j) * 8;
            av[u] = load16(k < half_k ? erow + k : hrow + k);
          }
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int ss = min(s + u, slast);
            const u32x4 x = load_a16<bf16_t, MODE>(a, mclamp, 4 * ss + j, inv);
            av[u] = (s + u < ks1 && xvalid) ? x : zero;
          }
        }
      };
      if constexpr (MODE != AMode::Gather) load_a();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ss = min(s + u, slast);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if constexpr (PACKED)
              bv[u][n][b] = __builtin_amdgcn_raw_buffer_load_b128(rs[n][b], (s + u - ks0) * 1024 + lane * 16, 0,
                                                                  kCachePolicyStream);
            else
              bv[u][n][b] = load16_stream(wp[n][b] + static_cast<int64_t>(ss) * WSTEP);
          }
      }
      if constexpr (MODE == AMode::Gather) load_a();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE == AMode::Gather) {
        // steps past the range and padding rows multiply zeros (applied only
        // now, so that no load waits for another)
#pragma unroll
        for (int u = 0; u < U; ++u) av[u] = (s + u < ks1 && xvalid) ? av[u] : zero;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[n][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                                __builtin_bit_cast(bf16x8, bv[u][n][b]), acc[n][b],
                                                                0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[wave][n * NB + b][lane] = acc[n][b];
    __syncthreads();
    const int t = g * NT + wave;
    if (wave < NT && t < T) {
      f32x4 sum[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        sum[b] = red[0][wave * NB + b][lane];
#pragma unroll
        for (int w = 1; w < SK; ++w) sum[b] += red[w][wave * NB + b][lane];
      }
      const int c = lane & 15;
      const int n = tile_row<EPI>(a, t, c);
      if constexpr (EPI == Epi::Store || EPI == Epi::AddTo) {
        if (splits > 1) {
          float* pz = a.part + static_cast<int64_t>(z) * a.M * a.ldy;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = 4 * j + q;
            if (m < a.M && n < a.Nout) pz[static_cast<int64_t>(m) * a.ldy + n] = sum[0][q];
          }
        } else {
          float sq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = 4 * j + q;
            float v = sum[0][q];
            sq[q] = 0.f;
            if (m < a.M && n < a.Nout) {
              float* y = a.y + static_cast<int64_t>(m) * a.ldy + n;
              if constexpr (EPI == Epi::AddTo) v += *y;
              *y = v;
              sq[q] = v * v;
            }
          }
          if (a.ss_out) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
              for (int off = 8; off >= 1; off >>= 1) sq[q] += __shfl_xor(sq[q], off, 64);
              const int m = 4 * j + q;
              if (c == 0 && m < a.M) a.ss_out[static_cast<int64_t>(t) * a.M + m] = sq[q];
            }
          }
        }
      } else if constexpr (EPI == Epi::SiluMul) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 4 * j + q;
          if (m >= a.M || n >= a.Nout) continue;
          const float v = sum[0][q];
          const float sg = v / (1.f + expf(-v));
          static_cast<bf16_t*>(a.y_op)[static_cast<int64_t>(m) * a.ldy + n] = f32_to_bf16(sg * sum[NB - 1][q]);
        }
      } else if constexpr (EPI == Epi::Argmax) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 4 * j + q;
          if (m >= a.M || n >= a.Nout) continue;
          const float v = sum[0][q];
          if (a.logits) a.logits[static_cast<int64_t>(m) * a.Nout + n] = v;
          top2_push(best[q], v, n);
        }
      } else {  // QkvRope
        const RopeOut& ro = a.rope;
        const int d = ro.d;
        const int head = n / d;
        const int e = n - head * d;                  // element within the head
        const bool rotate = head < ro.n_q + ro.n_kv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 4 * j + q;
          const float v = sum[0][q];
          const float partner = __shfl_xor(v, 8, 64);
          if (!r_live[q]) continue;
          float out = v;
          if (rotate) out = c < 8 ? v * rot[q].x - partner * rot[q].y : v * rot[q].x + partner * rot[q].y;
          if (head < ro.n_q) {
            static_cast<bf16_t*>(ro.q_out)[(static_cast<int64_t>(m) * ro.n_q + head) * d + e] = f32_to_bf16(out);
          } else {
            const int64_t slot = r_slot[q];
            if (slot < 0) continue;
            const bool is_k = head < ro.n_q + ro.n_kv;
            const int gg = is_k ? head - ro.n_q : head - ro.n_q - ro.n_kv;
            // 16-token pages (the only page size the library accepts)
            const int64_t blk = slot >> 4;
            const int off = static_cast<int>(slot & 15);
            static_cast<bf16_t*>(is_k ? ro.k_cache : ro.v_cache)[((blk * ro.n_kv + gg) * 16 + off) * d + e] =
                f32_to_bf16(out);
          }
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
        const int m = 4 * j + q;
        if ((lane & 15) == 0 && m < a.M) a.partials[static_cast<int64_t>(m) * gridDim.x + blockIdx.x] = best[q];
      }
    }
  }
}

// Packed copy: fragment (t, s) of W is 64 16-byte pieces, piece l holding
// W[row(t, l % 16)][32 s + 8 (l / 16) .. + 8] (zeros past the last row).
__global__ __launch_bounds__(256) void pack_kernel(PackArgs p) {
  const int64_t piece = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int KS = p.K / 32;
  const int64_t pieces = static_cast<int64_t>((p.Nout + 15) / 16) * KS * 64;
  if (piece >= pieces) return;
  const int lane = static_cast<int>(piece & 63);
  const int64_t frag = piece >> 6;
  const int t = static_cast<int>(frag / KS);
  const int s = static_cast<int>(frag - static_cast<int64_t>(t) * KS);
  const int c = lane & 15;
  const int row = p.rope_d > 0 ? rope_tile_row(t, c, p.rope_d) : t * 16 + c;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < p.Nout) {
    const bf16_t* src;
    if (row < p.n_a)
      src = static_cast<const bf16_t*>(p.w_a) + static_cast<int64_t>(row) * p.K;
    else if (row < p.n_a + p.n_b)
      src = static_cast<const bf16_t*>(p.w_b) + static_cast<int64_t>(row - p.n_a) * p.K;
    else
      src = static_cast<const bf16_t*>(p.w_c) + static_cast<int64_t>(row - p.n_a - p.n_b) * p.K;
    v = load16(src + s * 32 + (lane >> 4) * 8);
  }
  store16(static_cast<bf16_t*>(p.dst) + piece * 8, v);
}

// ------------------------------------------------------------------ dispatch
// Smallest activation-row tile that covers M (one pass over the weights),
// 16-row slices beyond that.  The bf16 LM head over 3..8 rows takes the 8-row
// tile, whose launch shape streams the vocabulary fastest (its padding rows
// cost VALU time only): 182 against 201 us over 3 rows at V = 201088.
int gemv_m_tile(int M, Epi epi, DType dt) {
  if (epi == Epi::Argmax && dt == DType::BF16 && M >= 3 && M <= 8) return 8;
  return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
}

// bf16 projections of up to 16 rows stream their weights through the MFMA
// kernel (padding rows of the 16-row fragment cost nothing at the HBM rate);
// the LM head over at most 8 rows keeps the LDS kernel, which streams its
// row-major weights fastest.
bool use_mfma(int M, int K, DType dt, Epi epi) {
  return dt == DType::BF16 && M >= 1 && M <= 16 && K % 32 == 0 && (epi != Epi::Argmax || M > 8);
}

// Launch shape of the weight-streaming MFMA kernel.
//   * Row-major weights, or epilogues that need whole sums in one workgroup
//     with few tiles: one tile per wave group, SK waves enough that each
//     wave's share of K is one batch of 12 k-steps (at most 8 waves for the
//     paired gate/up tiles, the argmax state and the RoPE epilogue).
//   * Packed weights with >= 320 tiles: two tiles per workgroup.
//   * Packed Store / AddTo whose consumer adds split partials: four tiles per
//     workgroup and K split over enough workgroups to cover most of the CUs.
struct SkinnyCfg {
  int sk, nt, u, splits;
};
SkinnyCfg skinny_cfg(const GemvArgs& a, Epi epi, int num_cus) {
  const int ks = a.K / 32;
  const int T = (a.Nout + 15) / 16;
  const bool packed = a.pk_a != nullptr && epi != Epi::Argmax;
  const bool whole = epi == Epi::Store || epi == Epi::AddTo;
  if (packed && whole && a.part && !a.ss_out) {
    // enough splits that each wave's share is one batch of 6 k-steps, and at
    // least enough workgroups for three quarters of the CUs
    const int groups = (T + 3) / 4;
    int sp = (ks + 8 * 6 - 1) / (8 * 6);
    const int fill = (num_cus * 3 / 4) / groups;
    if (sp < fill) sp = fill;
    const int max_sp = ks / 8;  // at least one k-step per wave
    if (sp > max_sp) sp = max_sp;
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp >= 2) return {8, 4, 6, sp};
  }
  if (packed && T >= 320 && ks >= 16) {
    // the paired gate/up tiles and the RoPE epilogue need 8-wave register
    // budgets; q/k/v keeps 12 k-steps per batch
    if (epi == Epi::SiluMul) return {8, 2, 6, 1};
    if (epi == Epi::QkvRope) return {8, 2, 12, 1};
    return {16, 2, 6, 1};
  }
  int sk = ks <= 48 ? 4 : ks <= 96 ? 8 : 16;
  if (!whole && sk > 8) sk = 8;
  return {sk, 1, 12, 1};
}

template <int SK, int NT, int U, Epi EPI, AMode MODE, bool PACKED>
hipError_t launch_skinny_t(GemvArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((mfma_skinny_kernel<SK, NT, U, EPI, MODE, PACKED>), grid, dim3(64 * SK), 0, s, a);
  return hipGetLastError();
}

template <Epi EPI, AMode MODE>
hipError_t launch_mfma(GemvArgs& a, int num_cus, hipStream_t s) {
  const SkinnyCfg cfg = skinny_cfg(a, EPI, num_cus);
  const int T = (a.Nout + 15) / 16;
  const int G = (T + cfg.nt - 1) / cfg.nt;
  const int gx = G < num_cus * 4 ? G : num_cus * 4;
  a.grid_x = gx;
  a.splits = cfg.splits;
  dim3 grid(gx, cfg.splits);
  constexpr bool rowmajor_only = EPI == Epi::Argmax;
  if (a.pk_a && !rowmajor_only) {
    if (cfg.nt == 4) {
      if constexpr (EPI == Epi::Store || EPI == Epi::AddTo) return launch_skinny_t<8, 4, 6, EPI, MODE, true>(a, grid, s);
      return hipErrorInvalidValue;
    }
    if (cfg.nt == 2) {
      if constexpr (EPI == Epi::SiluMul)
        return launch_skinny_t<8, 2, 6, EPI, MODE, true>(a, grid, s);
      else if constexpr (EPI == Epi::QkvRope)
        return launch_skinny_t<8, 2, 12, EPI, MODE, true>(a, grid, s);
      else if constexpr (EPI != Epi::Argmax) return launch_skinny_t<16, 2, 6, EPI, MODE, true>(a, grid, s);
      return hipErrorInvalidValue;
    }
    if constexpr (!rowmajor_only) {
      switch (cfg.sk) {
        case 16:
          if constexpr (EPI == Epi::Store || EPI == Epi::AddTo)
            return launch_skinny_t<16, 1, 12, EPI, MODE, true>(a, grid, s);
          return hipErrorInvalidValue;
        case 8: return launch_skinny_t<8, 1, 12, EPI, MODE, true>(a, grid, s);
        default: return launch_skinny_t<4, 1, 12, EPI, MODE, true>(a, grid, s);
      }
    }
  }
  switch (cfg.sk) {
    case 16:
      if constexpr (EPI == Epi::Store || EPI == Epi::AddTo) return launch_skinny_t<16, 1, 12, EPI, MODE, false>(a, grid, s);
      return hipErrorInvalidValue;
    case 8: return launch_skinny_t<8, 1, 12, EPI, MODE, false>(a, grid, s);
    default: return launch_skinny_t<4, 1, 12, EPI, MODE, false>(a, grid, s);
  }
}

template <typename TW, int MT, int R, Epi EPI, AMode MODE, int JS = 2>
hipError_t launch_lds(GemvArgs& a, dim3 grid, hipStream_t s) {
  const size_t lds = static_cast<size_t>(MT) * a.K * sizeof(TW);
  static bool raised = false;
  if (lds > 64 * 1024 && !raised) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_lds_kernel<TW, MT, R, EPI, MODE, JS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return hipErrorInvalidValue;
    raised = true;
  }
  hipLaunchKernelGGL((gemv_lds_kernel<TW, MT, R, EPI, MODE, JS>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <typename TW, Epi EPI, AMode MODE>
hipError_t launch_valu(GemvArgs& a, int num_cus, hipStream_t s) {
  const int m_tile = gemv_m_tile(a.M, EPI, sizeof(TW) == 2 ? DType::BF16 : DType::F32);
  const int R = m_tile >= 16 ? 4 : m_tile >= 8 ? 8 : 16;  // R * MT <= 64
  const int rg = EPI == Epi::SiluMul ? R / 2 : R;
  const int groups = (a.Nout + rg - 1) / rg;
  int gx = (groups + 3) / 4;
  if (gx > 2 * num_cus) gx = 2 * num_cus;
  if (gx < 1) gx = 1;
  a.grid_x = gx;
  dim3 grid(gx, (a.M + m_tile - 1) / m_tile);
  switch (m_tile) {
    case 16: return launch_lds<TW, 16, 4, EPI, MODE>(a, grid, s);
    // one k-step of the 8 weight rows in flight keeps this tile near 150
    // VGPRs (three waves per SIMD), which streams faster than two steps at
    // ~235 VGPRs and two waves per SIMD
    case 8: return launch_lds<TW, 8, 8, EPI, MODE, 1>(a, grid, s);
    case 4: return launch_lds<TW, 4, 16, EPI, MODE>(a, grid, s);
    case 2: return launch_lds<TW, 2, 16, EPI, MODE>(a, grid, s);
    default: return launch_lds<TW, 1, 16, EPI, MODE>(a, grid, s);
  }
}

}  // namespace

ProjKernel proj_kernel(int M, int K, DType dt, Epi epi) {
  if (dt == DType::BF16 && M > 16 && K % 64 == 0) return ProjKernel::Tiled;
  if (use_mfma(M, K, dt, epi)) return ProjKernel::Skinny;
  return ProjKernel::Lds;
}

bool gemv_uses_mfma(int M, int K, DType dt) { return proj_kernel(M, K, dt) != ProjKernel::Lds; }

int gemv_grid_x(int M, int Nout, Epi epi, DType dt, int num_cus, int K) {
  if (proj_kernel(M, K, dt, epi) == ProjKernel::Tiled) return gemm_parts(M, Nout, num_cus);
  if (use_mfma(M, K, dt, epi)) {
    // the argmax epilogue always runs one tile per group on row-major weights
    const int T = (Nout + 15) / 16;
    return T < num_cus * 4 ? T : num_cus * 4;
  }
  const int m_tile = gemv_m_tile(M, epi, dt);
  const int R = m_tile >= 16 ? 4 : m_tile >= 8 ? 8 : 16;
  const int rg = epi == Epi::SiluMul ? R / 2 : R;
  int gx = ((Nout + rg - 1) / rg + 3) / 4;
  if (gx > 2 * num_cus) gx = 2 * num_cus;
  return gx < 1 ? 1 : gx;
}

size_t gemv_lds_bytes(int M, int K, DType dt, Epi epi) {
  if (proj_kernel(M, K, dt, epi) != ProjKernel::Lds) return 0;
  return static_cast<size_t>(gemv_m_tile(M, epi, dt)) * K * elem_bytes(dt);
}

// Supported (epilogue, operand) pairs: every epilogue with a plain operand on
// the MFMA kernel (QkvRope only there), every epilogue but QkvRope with a plain
// operand on the LDS kernel; the fused forms Store+Gather (fc) and Argmax+Norm
// on the MFMA kernel, Argmax+Norm on the LDS kernel.
hipError_t launch_gemv(GemvArgs& a, Epi epi, DType dt, int num_cus, hipStream_t s) {
  a.splits = 1;
  if (epi == Epi::QkvRope && !a.rope.table) return hipErrorInvalidValue;
  if (proj_kernel(a.M, a.K, dt, epi) == ProjKernel::Tiled) return launch_gemm(a, epi, num_cus, s);
  // tile-major operands and outputs are read and written by the tiled kernels only
  if (a.x_group || a.y_group || (a.pk_tiles && epi != Epi::Argmax)) return hipErrorInvalidValue;
  if (use_mfma(a.M, a.K, dt, epi)) {
    if (a.amode == AMode::Plain) {
      switch (epi) {
        case Epi::Store: return launch_mfma<Epi::Store, AMode::Plain>(a, num_cus, s);
        case Epi::AddTo: return launch_mfma<Epi::AddTo, AMode::Plain>(a, num_cus, s);
        case Epi::SiluMul: return launch_mfma<Epi::SiluMul, AMode::Plain>(a, num_cus, s);
        case Epi::Argmax: return launch_mfma<Epi::Argmax, AMode::Plain>(a, num_cus, s);
        case Epi::QkvRope: return launch_mfma<Epi::QkvRope, AMode::Plain>(a, num_cus, s);
      }
      return hipErrorInvalidValue;
    }
    if (a.amode == AMode::Gather && epi == Epi::Store) return launch_mfma<Epi::Store, AMode::Gather>(a, num_cus, s);
    if (a.amode == AMode::Norm && epi == Epi::Argmax) return launch_mfma<Epi::Argmax, AMode::Norm>(a, num_cus, s);
    return hipErrorInvalidValue;
  }
  if (a.amode == AMode::Plain) {
    switch (epi) {
      case Epi::Store:
        return dt == DType::F32 ? launch_valu<float, Epi::Store, AMode::Plain>(a, num_cus, s)
                                : launch_valu<bf16_t, Epi::Store, AMode::Plain>(a, num_cus, s);
      case Epi::AddTo:
        return dt == DType::F32 ? launch_valu<float, Epi::AddTo, AMode::Plain>(a, num_cus, s)
                                : launch_valu<bf16_t, Epi::AddTo, AMode::Plain>(a, num_cus, s);
      case Epi::SiluMul:
        return dt == DType::F32 ? launch_valu<float, Epi::SiluMul, AMode::Plain>(a, num_cus, s)
                                : launch_valu<bf16_t, Epi::SiluMul, AMode::Plain>(a, num_cus, s);
      case Epi::Argmax:
        return dt == DType::F32 ? launch_valu<float, Epi::Argmax, AMode::Plain>(a, num_cus, s)
                                : launch_valu<bf16_t, Epi::Argmax, AMode::Plain>(a, num_cus, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.amode == AMode::Norm && epi == Epi::Argmax)
    return dt == DType::F32 ? launch_valu<float, Epi::Argmax, AMode::Norm>(a, num_cus, s)
                            : launch_valu<bf16_t, Epi::Argmax, AMode::Norm>(a, num_cus, s);
  return hipErrorInvalidValue;
}

size_t packed_bytes(int Nout, int K) { return static_cast<size_t>((Nout + 15) / 16) * 16 * K * 2; }

hipError_t launch_pack(const PackArgs& p, hipStream_t s) {
  if (p.K % 32 != 0 || p.Nout <= 0) return hipErrorInvalidValue;
  const int64_t pieces = static_cast<int64_t>((p.Nout + 15) / 16) * (p.K / 32) * 64;
  const int64_t blocks = (pieces + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pe
