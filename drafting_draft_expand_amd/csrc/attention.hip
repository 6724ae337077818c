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

// out[row, h, :] = sum_s acc_s * e^{m_s - M} / sum_s l_s * e^{m_s - M}
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int row = blockIdx.x;
  const int D = a.d;
  T* out = static_cast<T*>(a.out) + static_cast<int64_t>(row) * a.n_q * D;
  const bool rej = a.rejected[row];
  for (int e = threadIdx.x; e < a.n_q * D; e += blockDim.x) {
    const int h = e / D, dd = e - h * D;
    float res = 0.f;
    if (!rej) {
      const float* p = a.partial + (static_cast<int64_t>(row) * a.n_q + h) * a.splits * (D + 2);
      float M = -INFINITY;
      for (int s = 0; s < a.splits; ++s) M = fmaxf(M, p[s * (D + 2) + D]);
      float num = 0.f, den = 0.f;
      for (int s = 0; s < a.splits; ++s) {
        const float ms = p[s * (D + 2) + D];
        if (ms == -INFINITY) continue;
        const float w = expf(ms - M);
        num = fmaf(p[s * (D + 2) + dd], w, num);
        den = fmaf(p[s * (D + 2) + D + 1], w, den);
      }
      res = num / den;
    }
    out[e] = Elem<T>::from_f32(res);
  }
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.n_kv, a.c);
  switch (a.d) {
    case 16: hipLaunchKernelGGL((attn_split_kernel<T, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((attn_split_kernel<T, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((attn_split_kernel<T, 64>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_split_kernel<T, 128>), grid, dim3(256), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  return a.dtype == DType::F32 ? launch_t<float>(a, s) : launch_t<bf16_t>(a, s);
}

}  // namespace pe
