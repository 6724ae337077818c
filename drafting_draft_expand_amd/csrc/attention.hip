// Paged grouped-query attention of the draft rows, split over the KV range.
//
// Every non-rejected draft row at position p attends to positions 0..p of its
// own sequence (the cached context plus the rows this pass just wrote), with
// q head h reading kv head h / (n_q / n_kv).  The causal mask compares
// POSITIONS, not row indices: MASK rows sit at positions after the bonus row
// while rejected rows keep older positions and are skipped entirely.
//
// Grid (split, kv head, sequence).  A workgroup owns all query heads of one
// kv-head group for every row of its sequence, and one contiguous slice of the
// sequence's key positions; 64-key K/V tiles are gathered page by page into LDS
// (fp32) and scored against a 64-query tile kept in LDS, with an fp32 online
// softmax.  Each (row, head, split) leaves (acc[d], max, sum) in the workspace
// and a second kernel merges the splits with their log-sum-exp weights and
// stores the attention output as the next projection's operand.
#include "common.h"

namespace pe {
namespace {

constexpr int QT = 64;  // queries per tile
constexpr int KT = 64;  // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  __shared__ float qs[QT][D + 1];
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[KT][D + 1];
  __shared__ float sc[QT][KT + 1];
  __shared__ int qpos[QT];
  const int tid = threadIdx.x;
  const int sp = blockIdx.x, g = blockIdx.y, i = blockIdx.z;
  const int grp = a.n_q / a.n_kv;
  const int r0 = a.cu_draft[i], r1 = a.cu_draft[i + 1];
  const int kvlen = a.kv_lens[i];
  const int chunk = ((kvlen + a.splits - 1) / a.splits + 15) / 16 * 16;
  const int kb = sp * chunk;
  const int ke = min(kvlen, kb + chunk);
  const int nqry = (r1 - r0) * grp;
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  const T* qin = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
  constexpr int DP = D / 4;  // dims per thread in the PV update

  for (int qt0 = 0; qt0 < nqry; qt0 += QT) {
    for (int e = tid; e < QT * D; e += 256) {
      const int qi = e / D, dd = e - qi * D;
      const int q = qt0 + qi;
      float v = 0.f;
      if (q < nqry) {
        const int row = r0 + q / grp, h = g * grp + q % grp;
        v = Elem<T>::to_f32(qin[(static_cast<int64_t>(row) * a.n_q + h) * D + dd]) * scale;
      }
      qs[qi][dd] = v;
    }
    if (tid < QT) {
      const int q = qt0 + tid;
      int p = -1;  // -1: inactive query (past the end or rejected row)
      if (q < nqry) {
        const int row = r0 + q / grp;
        if (!a.rejected[row]) p = a.pos[row];
      }
      qpos[tid] = p;
    }
    const int qi = tid >> 2, part = tid & 3;
    float m_run = -INFINITY, l_run = 0.f;
    float acc[DP];
#pragma unroll
    for (int x = 0; x < DP; ++x) acc[x] = 0.f;
    __syncthreads();

    for (int kt0 = kb; kt0 < ke; kt0 += KT) {
      for (int e = tid; e < KT * D; e += 256) {
        const int kk = e / D, dd = e - kk * D;
        const int p = kt0 + kk;
        float kv = 0.f, vv = 0.f;
        if (p < ke) {
          const int64_t blk = bt[p / a.block_size];
          const int64_t base = ((blk * a.n_kv + g) * a.block_size + p % a.block_size) * D + dd;
          kv = Elem<T>::to_f32(kc[base]);
          vv = Elem<T>::to_f32(vc[base]);
        }
        ks[kk][dd] = kv;
        vs[kk][dd] = vv;
      }
      __syncthreads();
      {
        const int q2 = tid & 63;
        const int k0 = (tid >> 6) * 16;
        const int qp = qpos[q2];
        for (int kk = 0; kk < 16; ++kk) {
          const int key = k0 + kk;
          const int p = kt0 + key;
          float s = -INFINITY;
          if (p < ke && p <= qp) {
            s = 0.f;
#pragma unroll 16
            for (int dd = 0; dd < D; ++dd) s = fmaf(qs[q2][dd], ks[key][dd], s);
          }
          sc[q2][key] = s;
        }
      }
      __syncthreads();
      {
        float mx = -INFINITY;
        for (int kk = 0; kk < KT; ++kk) mx = fmaxf(mx, sc[qi][kk]);
        const float mnew = fmaxf(m_run, mx);
        if (mnew != -INFINITY) {
          const float corr = m_run == -INFINITY ? 0.f : expf(m_run - mnew);
          l_run *= corr;
#pragma unroll
          for (int x = 0; x < DP; ++x) acc[x] *= corr;
          for (int kk = 0; kk < KT; ++kk) {
            const float s = sc[qi][kk];
            if (s == -INFINITY) continue;
            const float pr = expf(s - mnew);
            l_run += pr;
#pragma unroll
            for (int x = 0; x < DP; ++x) acc[x] = fmaf(pr, vs[kk][part * DP + x], acc[x]);
          }
          m_run = mnew;
        }
      }
      __syncthreads();
    }

    const int q = qt0 + qi;
    if (q < nqry) {
      const int row = r0 + q / grp, h = g * grp + q % grp;
      float* o = a.partial + ((static_cast<int64_t>(row) * a.n_q + h) * a.splits + sp) * (D + 2);
#pragma unroll
      for (int x = 0; x < DP; ++x) o[part * DP + x] = acc[x];
      if (part == 0) {
        o[D] = m_run;
        o[D + 1] = l_run;
      }
    }
    __syncthreads();
  }
}

// bf16, head_dim 64/128: the same split-KV attention on MFMA.
//
// A workgroup of 8 waves owns up to 128 queries (16 per wave) of one
// (sequence, kv head, split).  Per 64-key tile the waves share K (row-major)
// and V (transposed) in LDS.  Scores are formed transposed, S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (keys are the A rows, the wave's queries the B
// columns), so each lane owns one query column: the online-softmax row
// statistics need only the 4 lanes that share that column, and the
// probabilities are already in the B-operand layout of O^T += V^T P^T.  In
// that product the MFMA's 32 k-slots of each 32-key half enumerate keys
// 4j..4j+3 and 16+4j..16+4j+3 for lane group j, the order in which the score
// tiles hold them.  K/V pieces of the next two tiles are kept in flight in
// registers while the current tile is consumed from LDS.
template <int D>
__global__ __launch_bounds__(512) void attn_mfma_kernel(AttnArgs a) {
  constexpr int KT = 64;
  constexpr int KP = D + 8;    // padded K row (elements)
  constexpr int VP = KT + 8;   // padded V^T row (elements)
  constexpr int DT = D / 16;   // O^T tiles
  constexpr int KK = D / 32;   // k-steps of S^T
  constexpr int PER = KT * D / 8 / 512;  // 16-byte K (and V) pieces per thread per tile
  static_assert(PER >= 1, "tile too small for the workgroup");
  constexpr int MAXB = 1024;   // pages of one split held in LDS
  __shared__ bf16_t ks[KT * KP];
  __shared__ bf16_t vt[D * VP];
  __shared__ int32_t pages[MAXB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, j = lane >> 4;
  const int sp = blockIdx.x, g = blockIdx.y, i = blockIdx.z;
  const int grp = a.n_q / a.n_kv;
  const int r0 = a.cu_draft[i], r1 = a.cu_draft[i + 1];
  const int kvlen = a.kv_lens[i];
  const int chunk = ((kvlen + a.splits - 1) / a.splits + KT - 1) / KT * KT;
  const int kb = sp * chunk;
  const int ke = min(kvlen, kb + chunk);
  const int ntiles = ke > kb ? (ke - kb + KT - 1) / KT : 0;
  const int nqry = (r1 - r0) * grp;
  const float sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));  // scale * log2(e)
  const bf16_t* qin = static_cast<const bf16_t*>(a.q);
  const bf16_t* kc = static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vc = static_cast<const bf16_t*>(a.v_cache);
  const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // the split's page numbers, so K/V addresses do not wait on a table load
  const int pg0 = kb / a.block_size;
  const int npg = ke > kb ? (ke - 1) / a.block_size - pg0 + 1 : 0;
  const bool paged_lds = npg <= MAXB;
  for (int q = tid; q < npg && paged_lds; q += 512) pages[q] = bt[pg0 + q];
  __syncthreads();

  constexpr int DEPTH = 3;  // tiles in flight
  u32x4 kr[DEPTH][PER], vr[DEPTH][PER];
  auto fetch = [&](int t, int set) {
#pragma unroll
    for (int pp = 0; pp < PER; ++pp) {
      const int piece = tid + 512 * pp;
      const int key = piece / (D / 8), c8 = piece % (D / 8);
      const int p = kb + t * KT + key;
      kr[set][pp] = zero;
      vr[set][pp] = zero;
      if (p < ke) {
        const int64_t blk = paged_lds ? pages[p / a.block_size - pg0] : bt[p / a.block_size];
        const int64_t off = ((blk * a.n_kv + g) * a.block_size + p % a.block_size) * D + c8 * 8;
        kr[set][pp] = load16(kc + off);
        vr[set][pp] = load16(vc + off);
      }
    }
  };
  auto stash = [&](int set) {
#pragma unroll
    for (int pp = 0; pp < PER; ++pp) {
      const int piece = tid + 512 * pp;
      const int key = piece / (D / 8), c8 = piece % (D / 8);
      store16(ks + key * KP + c8 * 8, kr[set][pp]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = vr[set][pp][e];
        vt[(c8 * 8 + 2 * e) * VP + key] = static_cast<bf16_t>(w & 0xffffu);
        vt[(c8 * 8 + 2 * e + 1) * VP + key] = static_cast<bf16_t>(w >> 16);
      }
    }
  };

  for (int qb = 0; qb < nqry; qb += 128) {
    const int qn = qb + wave * 16 + (lane & 15);
    const int row = r0 + qn / grp;
    const int h = g * grp + qn % grp;
    const bool active = qn < nqry && !a.rejected[row];
    const int qpos = active ? a.pos[row] : -1;
    u32x4 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = active ? load16(qin + (static_cast<int64_t>(row) * a.n_q + h) * D + 32 * kk + 8 * j) : zero;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int t = 0; t < DEPTH; ++t)
      if (t < ntiles) fetch(t, t);
    for (int t = 0; t < ntiles; ++t) {
      const int kt0 = kb + t * KT;
      const int set = t % DEPTH;
      __syncthreads();
      stash(set);
      __syncthreads();
      if (t + DEPTH < ntiles) fetch(t + DEPTH, set);

      f32x4 st[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 af = *reinterpret_cast<const u32x4*>(ks + (mt * 16 + (lane & 15)) * KP + 32 * kk + 8 * j);
          st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                           __builtin_bit_cast(bf16x8, qf[kk]), st[mt], 0, 0, 0);
        }
      }
      float sv[16];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = kt0 + mt * 16 + 4 * j + q;
          const float sc = (p < ke && p <= qpos) ? st[mt][q] * sl2 : -INFINITY;
          sv[mt * 4 + q] = sc;
          mx = fmaxf(mx, sc);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float corr = m_run == -INFINITY ? (m_new == -INFINITY ? 1.f : 0.f) : exp2f(m_run - m_new);
      float rs = 0.f;
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p0 = sv[2 * e] == -INFINITY ? 0.f : exp2f(sv[2 * e] - m_new);
        const float p1 = sv[2 * e + 1] == -INFINITY ? 0.f : exp2f(sv[2 * e + 1] - m_new);
        rs += p0 + p1;
        pk[e] = static_cast<uint32_t>(f32_to_bf16(p0)) | (static_cast<uint32_t>(f32_to_bf16(p1)) << 16);
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * corr + rs;
      m_run = m_new;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 pb = {pk[4 * hf], pk[4 * hf + 1], pk[4 * hf + 2], pk[4 * hf + 3]};
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) {
          if (hf == 0) o[t2] *= corr;
          const bf16_t* vr_ = vt + (t2 * 16 + (lane & 15)) * VP + hf * 32;
          const uint2 lo = *reinterpret_cast<const uint2*>(vr_ + 4 * j);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr_ + 16 + 4 * j);
          const u32x4 af = {lo.x, lo.y, hi.x, hi.y};
          o[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                          __builtin_bit_cast(bf16x8, pb), o[t2], 0, 0, 0);
        }
      }
    }
    if (qn < nqry && !a.rejected[row]) {
      float* out = a.partial + ((static_cast<int64_t>(row) * a.n_q + h) * a.splits + sp) * (D + 2);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) out[t * 16 + 4 * j + q] = o[t][q];
      if (j == 0) {
        // row statistics in natural-log units for the combine step
        out[D] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
        out[D + 1] = l_run;
      }
    }
    __syncthreads();
  }
}

// out[row, h, :] = sum_s acc_s * e^{m_s - M} / sum_s l_s * e^{m_s - M};
// one 64-thread workgroup per (row, head), split weights shared through LDS.
template <typename T>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wgt[64];
  const int row = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int D = a.d, S = a.splits;
  T* out = static_cast<T*>(a.out) + (static_cast<int64_t>(row) * a.n_q + h) * D;
  if (a.rejected[row]) {
    for (int dd = lane; dd < D; dd += 64) out[dd] = Elem<T>::from_f32(0.f);
    return;
  }
  const float* p = a.partial + (static_cast<int64_t>(row) * a.n_q + h) * S * (D + 2);
  const float ms = lane < S ? p[lane * (D + 2) + D] : -INFINITY;
  const float M = wave_max(ms);
  const float w = ms == -INFINITY ? 0.f : expf(ms - M);
  const float den = wave_sum(lane < S ? w * p[lane * (D + 2) + D + 1] : 0.f);
  wgt[lane] = w;
  __syncthreads();
  const float inv = 1.f / den;
  for (int dd = lane; dd < D; dd += 64) {
    float num = 0.f;
    for (int s = 0; s < S; ++s) num = fmaf(p[s * (D + 2) + dd], wgt[s], num);
    out[dd] = Elem<T>::from_f32(num * inv);
  }
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.n_kv, a.c);
  if (sizeof(T) == 2 && (a.d == 64 || a.d == 128)) {
    if (a.d == 64)
      hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(512), 0, s, a);
  } else {
    switch (a.d) {
      case 16: hipLaunchKernelGGL((attn_split_kernel<T, 16>), grid, dim3(256), 0, s, a); break;
      case 32: hipLaunchKernelGGL((attn_split_kernel<T, 32>), grid, dim3(256), 0, s, a); break;
      case 64: hipLaunchKernelGGL((attn_split_kernel<T, 64>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((attn_split_kernel<T, 128>), grid, dim3(256), 0, s, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(a.N, a.n_q), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  return a.dtype == DType::F32 ? launch_t<float>(a, s) : launch_t<bf16_t>(a, s);
}

}  // namespace pe
