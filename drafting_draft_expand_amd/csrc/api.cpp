// C ABI of the parallel-draft step: host-side validation, workspace layout and
// launch sequencing.  Declarations and argument contracts: include/peagle.h.
#include "../../include/peagle.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "internal.h"

using pe::DType;

namespace {

// Kernel timing for measurement harnesses: one process-wide record per kernel
// class, guarded by a mutex, so that the model handles stay read-only after
// set-up.  The event pairs are created on first use and reused until the
// process ends.
struct Timing {
  std::atomic<bool> enabled{false};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;  // recorded pairs
  size_t used = 0;
};
constexpr int kTimingClasses = 3;
std::mutex g_timing_mu;
Timing g_timing[kTimingClasses];

}  // namespace

// Packed copies of the projection weights (caller-owned buffer attached by
// pe_model_pack_weights): fragment order for the weight-streaming MFMA kernel
// (qkv .. down), tile-major in the ring's load order for passes over more
// than 256 rows (t_*, null when the shapes do not take that route).
struct PackedLayer {
  const void *qkv, *o, *gate, *up, *down;
  const void *t_qkv, *t_o, *t_gu, *t_down;
};

struct pe_model {
  pe_model_desc d;
  pe_weights w;
  std::vector<pe_layer_weights> layers;
  const void* pk_fc = nullptr;
  const void* pk_fc_tiles = nullptr;   // tile-major fc (passes over > 256 rows)
  std::vector<PackedLayer> pk_layers;  // empty: not packed
  const void* pk_lm = nullptr;         // tile-major LM head (packed models)
  int num_cus = 256;  // compute units of the device current at create
  pe::RopeFreq freq; // theta^(-2j/d) in double precision
};

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline DType dt(const pe_model* m) { return m->d.dtype == PE_F32 ? DType::F32 : DType::BF16; }

// KV-range splits per (sequence, kv head).  The bf16 LDS-ring kernels take
// the longest ranges first, so about two workgroups per slot suffice to
// balance the chip: 1024 for 64-dim heads (two workgroups per CU), 512 for
// 128-dim heads (one); fewer splits also mean less partial-result traffic.
// The other kernels take about 2048 workgroups (eight per CU) so that the
// per-tile softmax work of long contexts spreads over the chip.
int attention_splits(int c, int n_kv, int head_dim, pe_dtype dtype) {
  const int base = c * n_kv;
  const int target = dtype != PE_BF16 ? 2048 : head_dim == 64 ? 1024 : head_dim == 128 ? 512 : 2048;
  int s = (target + base - 1) / base;
  if (s < 1) s = 1;
  if (s > pe::kAttnMaxSplits) s = pe::kAttnMaxSplits;
  return s;
}

// Workspace carve-up for one forward call.
struct Workspace {
  size_t x, act, qkv, q, attn_part, mlp, top2, f, ss0, part, rope, total;
  int splits, lm_parts;
};

// Split partials of the projections that write the residual rows (the next
// RMSNorm adds them up).
inline size_t part_bytes(const pe_model_desc& d, int N) { return size_t(pe::kMaxSplits) * N * d.hidden * 4; }

Workspace plan_workspace(const pe_model* m, int c, int K, int N) {
  const pe_model_desc& d = m->d;
  const size_t eb = d.dtype == PE_F32 ? 4 : 2;
  const int S = c * K;
  const int H = d.hidden, qd = d.n_q * d.head_dim, kvd = d.n_kv * d.head_dim;
  int act_cols = 2 * H;
  if (qd > act_cols) act_cols = qd;
  if (d.inter > act_cols) act_cols = d.inter;
  Workspace w{};
  w.splits = attention_splits(c, d.n_kv, d.head_dim, d.dtype);
  w.lm_parts = 4096;  // upper bound on LM-head workgroups (grid is capped at 2 per CU)
  size_t off = 0;
  w.x = off;         off += align_up(size_t(N) * H * 4);
  // (act and mlp rounded up to 128 rows: over > 256 rows they may be written
  // tile-major in 128-row groups)
  const size_t Np = size_t(N + 127) / 128 * 128;
  w.act = off;       off += align_up(Np * act_cols * eb);
  w.qkv = off;       off += align_up(size_t(N) * (qd + 2 * kvd) * 4);
  w.q = off;         off += align_up(size_t(N) * qd * eb);
  w.attn_part = off; off += align_up(size_t(N) * d.n_q * w.splits * (d.head_dim + 2) * 4);
  w.mlp = off;       off += align_up(Np * d.inter * eb);
  w.top2 = off;      off += align_up(size_t(S) * w.lm_parts * sizeof(pe::Top2));
  // (rounded up to 128 rows: the LM head may read it tile-major in 128-row groups)
  w.f = off;         off += align_up(size_t((S + 127) / 128 * 128) * H * eb);
  w.ss0 = off;       off += align_up(size_t((H + 15) / 16) * N * 4);
  w.part = off;      off += align_up(part_bytes(d, N));
  w.rope = off;      off += align_up(size_t(N) * (d.head_dim / 2) * 2 * sizeof(float));
  w.total = off;
  return w;
}

pe_status check_desc(const pe_model_desc* d) {
  if (!d) return PE_EINVAL;
  if (d->hidden <= 0 || d->hidden % 8 != 0 || d->hidden > pe::kMaxHidden) return PE_EUNSUPPORTED;
  if (d->n_layers < 0 || d->block_size != 16) return PE_EUNSUPPORTED;
  if (d->dtype != PE_F32 && d->dtype != PE_BF16) return PE_EUNSUPPORTED;
  if (d->n_layers == 0) return PE_OK;  // expansion-only model
  if (d->vocab <= 0 || d->n_q <= 0 || d->n_kv <= 0 || d->n_q % d->n_kv != 0) return PE_EINVAL;
  if (d->head_dim != 16 && d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
    return PE_EUNSUPPORTED;
  if (d->inter <= 0 || d->inter % 8 != 0) return PE_EUNSUPPORTED;
  if ((d->n_q * d->head_dim) % 8 != 0) return PE_EUNSUPPORTED;
  if (d->mask_token_id < 0 || d->mask_token_id >= d->vocab) return PE_EINVAL;
  if (!(d->rms_eps > 0.f) || !(d->rope_theta > 0.f)) return PE_EINVAL;
  return PE_OK;
}

// Fused plan: every projection runs on the MFMA kernel, which gathers the fc
// input on the fly, applies RoPE + the KV write in the q/k/v epilogue and
// emits the row sums of squares the LM head needs for the final RMSNorm.
// Otherwise separate gather / RoPE / final-norm kernels are used.
bool fused_plan(const pe_model_desc& d, int N) {
  const pe::DType t = d.dtype == PE_F32 ? pe::DType::F32 : pe::DType::BF16;
  const int qd = d.n_q * d.head_dim;
  const int ks[] = {2 * d.hidden, d.hidden, qd, d.inter};
  for (int k : ks)
    if (!pe::gemv_uses_mfma(N, k, t)) return false;
  return d.hidden % 32 == 0 && d.head_dim % 16 == 0;
}

// The final RMSNorm rides in the LM head when the down projection emits row
// sums of squares (weight-streaming MFMA kernel) and the LM head stages its
// rows itself (LDS GEMV or weight-streaming MFMA).
bool fused_final_norm(const pe_model_desc& d, int N, int S) {
  const pe::DType t = d.dtype == PE_F32 ? pe::DType::F32 : pe::DType::BF16;
  return pe::proj_kernel(N, d.inter, t) == pe::ProjKernel::Skinny &&
         pe::proj_kernel(S, d.hidden, t) != pe::ProjKernel::Tiled;
}

// Compute units of the current device (256 if the runtime cannot say, e.g.
// on a host without a GPU, where nothing is launched anyway).
int query_num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  (void)hipGetLastError();  // leave no sticky error behind
  return 256;
}

// Optional event pair around one launch of a timed kernel class; while the
// class is enabled the scope holds the timing lock, so concurrent callers
// record their pairs one after the other.
struct TimedScope {
  Timing* t;
  hipStream_t s;
  hipEvent_t stop = nullptr;
  std::unique_lock<std::mutex> lock;
  TimedScope(pe_kernel_class k, hipStream_t stream, bool allowed = true) : t(&g_timing[k]), s(stream) {
    if (!allowed || !t->enabled.load(std::memory_order_relaxed)) { t = nullptr; return; }
    lock = std::unique_lock<std::mutex>(g_timing_mu);
    if (!t->enabled.load(std::memory_order_relaxed)) { t = nullptr; return; }
    if (t->used == t->events.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) { t = nullptr; return; }
      t->events.emplace_back(a, b);
    }
    (void)hipEventRecord(t->events[t->used].first, s);
    stop = t->events[t->used].second;
  }
  ~TimedScope() {
    if (!t) return;
    (void)hipEventRecord(stop, s);
    ++t->used;
  }
};

#define PE_HIP(expr)                                  \
  do {                                                \
    if ((expr) != hipSuccess) return PE_EHIP;          \
  } while (0)

}  // namespace

extern "C" {

const char* pe_status_string(pe_status s) {
  switch (s) {
    case PE_OK: return "ok";
    case PE_EINVAL: return "invalid argument";
    case PE_EUNSUPPORTED: return "unsupported shape or dtype";
    case PE_EWORKSPACE: return "workspace too small";
    case PE_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

pe_status pe_model_create(const pe_model_desc* desc, const pe_weights* w, pe_model** out) {
  if (!out || !w) return PE_EINVAL;
  *out = nullptr;
  pe_status st = check_desc(desc);
  if (st != PE_OK) return st;
  if (!w->h_shared || !aligned16(w->h_shared)) return PE_EINVAL;
  if (desc->n_layers > 0) {
    const void* req[] = {w->embed, w->w_fc, w->ln_f, w->w_lm};
    for (const void* p : req)
      if (!p || !aligned16(p)) return PE_EINVAL;
    if (!w->layers) return PE_EINVAL;
    for (int l = 0; l < desc->n_layers; ++l) {
      const pe_layer_weights& L = w->layers[l];
      const void* lp[] = {L.ln1, L.wq, L.wk, L.wv, L.wo, L.ln2, L.w_gate, L.w_up, L.w_down};
      for (const void* p : lp)
        if (!p || !aligned16(p)) return PE_EINVAL;
    }
  }
  pe_model* m = new (std::nothrow) pe_model();
  if (!m) return PE_EINVAL;
  m->d = *desc;
  m->w = *w;
  if (desc->n_layers > 0) m->layers.assign(w->layers, w->layers + desc->n_layers);
  for (int j = 0; j < 64; ++j)
    m->freq.inv[j] = desc->n_layers > 0 && j < desc->head_dim / 2
                         ? std::pow(static_cast<double>(desc->rope_theta), -2.0 * j / desc->head_dim)
                         : 0.0;
  m->w.layers = m->layers.empty() ? nullptr : m->layers.data();
  m->num_cus = query_num_cus();
  *out = m;
  return PE_OK;
}

void pe_model_destroy(pe_model* m) { delete m; }

namespace {
// The matrices the weight-streaming kernel reads, in buffer order: fc, then
// per layer q/k/v (RoPE pair order), o, gate, up, down.  Empty when the model
// has no bf16 layers or a dimension the kernel cannot take (K % 32).
void pack_plan(const pe_model* m, std::vector<pe::PackArgs>& v) {
  v.clear();
  const pe_model_desc& d = m->d;
  const int H = d.hidden, qd = d.n_q * d.head_dim, kvd = d.n_kv * d.head_dim, I = d.inter;
  if (d.dtype != PE_BF16 || d.n_layers <= 0) return;
  if (H % 32 != 0 || qd % 32 != 0 || I % 32 != 0 || d.head_dim % 16 != 0) return;
  auto one = [](const void* w, int nout, int k, int rope_d) {
    pe::PackArgs p{};
    p.w_a = p.w_b = p.w_c = w; p.n_a = nout; p.n_b = 0; p.Nout = nout; p.K = k; p.rope_d = rope_d;
    return p;
  };
  v.push_back(one(m->w.w_fc, H, 2 * H, 0));
  for (int l = 0; l < d.n_layers; ++l) {
    const pe_layer_weights& L = m->layers[l];
    pe::PackArgs q{};
    q.w_a = L.wq; q.w_b = L.wk; q.w_c = L.wv; q.n_a = qd; q.n_b = kvd; q.Nout = qd + 2 * kvd; q.K = H;
    q.rope_d = d.head_dim;
    v.push_back(q);
    v.push_back(one(L.wo, H, qd, 0));
    v.push_back(one(L.w_gate, I, H, 0));
    v.push_back(one(L.w_up, I, H, 0));
    v.push_back(one(L.w_down, H, I, 0));
  }
}
}  // namespace

namespace {
// Tile-major copies for the ring GEMM over more than 256 rows, in buffer
// order: fc, then per layer q/k/v, o, gate/up, down.  Only when every
// projection takes the tiled route there (bf16, each K a multiple of 64), as
// the producers of their operands then write them tile-major too.
bool many_rows_tiles(const pe_model_desc& d) {
  const int qd = d.n_q * d.head_dim;
  return d.dtype == PE_BF16 && d.n_layers > 0 && d.hidden % 64 == 0 && qd % 64 == 0 && d.inter % 64 == 0;
}
struct TileCopy {
  pe::Epi epi;
  pe::GemvArgs g;
};
void tile_plan(const pe_model* m, std::vector<TileCopy>& v) {
  v.clear();
  const pe_model_desc& d = m->d;
  if (!many_rows_tiles(d)) return;
  const int H = d.hidden, qd = d.n_q * d.head_dim, kvd = d.n_kv * d.head_dim, I = d.inter;
  auto one = [](pe::Epi e, const void* a, const void* b, const void* c, int n_a, int n_b, int nout, int k,
                int rope_d) {
    TileCopy t{};
    t.epi = e;
    t.g.w_a = a; t.g.w_b = b; t.g.w_c = c; t.g.n_a = n_a; t.g.n_b = n_b; t.g.Nout = nout; t.g.K = k;
    t.g.rope.d = rope_d;
    return t;
  };
  v.push_back(one(pe::Epi::Store, m->w.w_fc, m->w.w_fc, m->w.w_fc, H, 0, H, 2 * H, 0));
  for (int l = 0; l < d.n_layers; ++l) {
    const pe_layer_weights& L = m->layers[l];
    v.push_back(one(pe::Epi::QkvRope, L.wq, L.wk, L.wv, qd, kvd, qd + 2 * kvd, H, d.head_dim));
    v.push_back(one(pe::Epi::AddTo, L.wo, L.wo, L.wo, H, 0, H, qd, 0));
    v.push_back(one(pe::Epi::SiluMul, L.w_gate, L.w_up, L.w_up, I, I, I, H, 0));
    v.push_back(one(pe::Epi::AddTo, L.w_down, L.w_down, L.w_down, H, 0, H, I, 0));
  }
}
}  // namespace

size_t pe_packed_weights_bytes(const pe_model* m) {
  if (!m) return 0;
  size_t total = 0;
  std::vector<pe::PackArgs> plan;
  pack_plan(m, plan);
  for (const pe::PackArgs& p : plan) total += align_up(pe::packed_bytes(p.Nout, p.K));
  if (!plan.empty()) {
    total += align_up(pe::packed_tile_bytes(m->d.vocab, m->d.hidden));
    std::vector<TileCopy> tiles;
    tile_plan(m, tiles);
    for (const TileCopy& t : tiles) total += align_up(pe::proj_tile_bytes(t.epi, t.g.Nout, t.g.K));
  }
  return total;
}

pe_status pe_model_pack_weights(pe_model* m, void* packed, size_t packed_bytes, hipStream_t stream) {
  if (!m) return PE_EINVAL;
  std::vector<pe::PackArgs> plan;
  pack_plan(m, plan);
  if (plan.empty()) return PE_OK;
  if (!packed || (reinterpret_cast<uintptr_t>(packed) % kAlign) != 0) return PE_EINVAL;
  if (packed_bytes < pe_packed_weights_bytes(m)) return PE_EWORKSPACE;
  std::vector<const void*> dst;
  char* b = static_cast<char*>(packed);
  for (pe::PackArgs& p : plan) {
    p.dst = b;
    dst.push_back(b);
    PE_HIP(pe::launch_pack(p, stream));
    b += align_up(pe::packed_bytes(p.Nout, p.K));
  }
  PE_HIP(pe::launch_pack_tiles(m->w.w_lm, m->d.vocab, m->d.hidden, b, stream));
  const void* lm = b;
  b += align_up(pe::packed_tile_bytes(m->d.vocab, m->d.hidden));
  std::vector<TileCopy> tiles;
  tile_plan(m, tiles);
  std::vector<const void*> tdst;
  for (const TileCopy& t : tiles) {
    PE_HIP(pe::launch_pack_proj_tiles(t.epi, t.g, b, stream));
    tdst.push_back(b);
    b += align_up(pe::proj_tile_bytes(t.epi, t.g.Nout, t.g.K));
  }
  m->pk_lm = lm;
  m->pk_fc = dst[0];
  m->pk_fc_tiles = tdst.empty() ? nullptr : tdst[0];
  m->pk_layers.assign(m->d.n_layers, PackedLayer{});
  for (int l = 0; l < m->d.n_layers; ++l) {
    const void* const* q = dst.data() + 1 + 5 * l;
    PackedLayer P{q[0], q[1], q[2], q[3], q[4], nullptr, nullptr, nullptr, nullptr};
    if (!tdst.empty()) {
      const void* const* t = tdst.data() + 1 + 4 * l;
      P.t_qkv = t[0]; P.t_o = t[1]; P.t_gu = t[2]; P.t_down = t[3];
    }
    m->pk_layers[l] = P;
  }
  return PE_OK;
}

size_t pe_workspace_bytes(const pe_model* m, int32_t c, int32_t K, int32_t N) {
  if (!m || c <= 0 || K <= 0 || N <= 0 || m->d.n_layers <= 0) return 0;
  return plan_workspace(m, c, K, N).total;
}

namespace {
pe_status prepare_impl(const pe_model* m, int32_t c, int32_t K, int32_t T, const int32_t* query_lens,
                       const int32_t* target_ids, const int32_t* target_pos, const int32_t* num_accepted,
                       const int32_t* bonus_ids, const void* target_hidden, const int32_t* block_table,
                       int32_t max_blocks, int32_t* draft_ids, int32_t* draft_pos, int64_t* slot_mapping,
                       uint8_t* is_rejected, uint8_t* is_masked, int32_t* hidden_map, int32_t* cu_draft,
                       int32_t* kv_lens, int32_t* sample_idx, void* draft_hidden, hipStream_t stream,
                       int compact) {
  if (!m || c <= 0 || K <= 0 || T < c || max_blocks <= 0) return PE_EINVAL;
  const void* ptrs[] = {query_lens, target_ids, target_pos, num_accepted, bonus_ids, target_hidden,
                        block_table, draft_ids, draft_pos, slot_mapping, is_rejected, is_masked,
                        hidden_map, cu_draft, kv_lens, sample_idx, draft_hidden};
  for (const void* p : ptrs)
    if (!p) return PE_EINVAL;
  if (!aligned16(target_hidden) || !aligned16(draft_hidden)) return PE_EINVAL;
  const int64_t N = int64_t(T) + int64_t(c) * (K - 1);
  if (N > INT32_MAX) return PE_EINVAL;
  pe::PrepareArgs a{};
  a.c = c; a.K = K; a.T = T; a.N = int(N); a.H = m->d.hidden;
  a.block_size = m->d.block_size; a.max_blocks = max_blocks; a.mask_id = m->d.mask_token_id;
  a.dtype = dt(m);
  a.query_lens = query_lens; a.target_ids = target_ids; a.target_pos = target_pos;
  a.num_accepted = num_accepted; a.bonus_ids = bonus_ids; a.block_table = block_table;
  a.target_hidden = target_hidden; a.h_shared = m->w.h_shared;
  a.draft_ids = draft_ids; a.draft_pos = draft_pos; a.slot_mapping = slot_mapping;
  a.is_rejected = is_rejected; a.is_masked = is_masked; a.hidden_map = hidden_map;
  a.cu_draft = cu_draft; a.kv_lens = kv_lens; a.sample_idx = sample_idx; a.draft_hidden = draft_hidden;
  a.compact = compact;
  TimedScope ts(PE_KERNEL_PREPARE, stream);
  PE_HIP(pe::launch_prepare(a, stream));
  return PE_OK;
}
}  // namespace

pe_status pe_prepare_draft_batch(const pe_model* m, int32_t c, int32_t K, int32_t T,
                                 const int32_t* query_lens, const int32_t* target_ids,
                                 const int32_t* target_pos, const int32_t* num_accepted,
                                 const int32_t* bonus_ids, const void* target_hidden,
                                 const int32_t* block_table, int32_t max_blocks, int32_t* draft_ids,
                                 int32_t* draft_pos, int64_t* slot_mapping, uint8_t* is_rejected,
                                 uint8_t* is_masked, int32_t* hidden_map, int32_t* cu_draft,
                                 int32_t* kv_lens, int32_t* sample_idx, void* draft_hidden,
                                 hipStream_t stream) {
  return prepare_impl(m, c, K, T, query_lens, target_ids, target_pos, num_accepted, bonus_ids, target_hidden,
                      block_table, max_blocks, draft_ids, draft_pos, slot_mapping, is_rejected, is_masked,
                      hidden_map, cu_draft, kv_lens, sample_idx, draft_hidden, stream, 0);
}

pe_status pe_prepare_draft_batch_compact(const pe_model* m, int32_t c, int32_t K, int32_t T,
                                         const int32_t* query_lens, const int32_t* target_ids,
                                         const int32_t* target_pos, const int32_t* num_accepted,
                                         const int32_t* bonus_ids, const void* target_hidden,
                                         const int32_t* block_table, int32_t max_blocks, int32_t* draft_ids,
                                         int32_t* draft_pos, int64_t* slot_mapping, uint8_t* is_rejected,
                                         uint8_t* is_masked, int32_t* hidden_map, int32_t* cu_draft,
                                         int32_t* kv_lens, int32_t* sample_idx, void* draft_hidden,
                                         hipStream_t stream) {
  return prepare_impl(m, c, K, T, query_lens, target_ids, target_pos, num_accepted, bonus_ids, target_hidden,
                      block_table, max_blocks, draft_ids, draft_pos, slot_mapping, is_rejected, is_masked,
                      hidden_map, cu_draft, kv_lens, sample_idx, draft_hidden, stream, 1);
}

pe_status pe_check_verified_batch(const pe_model* m, int32_t c, int32_t K, int32_t T, const int32_t* query_lens,
                                  const int32_t* target_ids, const int32_t* target_pos, const int32_t* num_accepted,
                                  const int32_t* bonus_ids, const int32_t* block_table, int32_t max_blocks,
                                  int32_t* error_bits, hipStream_t stream) {
  if (!m || c <= 0 || K <= 0 || T < c || max_blocks <= 0) return PE_EINVAL;
  const void* ptrs[] = {query_lens, target_ids, target_pos, num_accepted, bonus_ids, block_table, error_bits};
  for (const void* p : ptrs)
    if (!p) return PE_EINVAL;
  static_assert(PE_CHECK_QUERY_LEN == pe::kCheckQueryLen && PE_CHECK_ACCEPTED == pe::kCheckAccepted &&
                    PE_CHECK_TOKEN_ID == pe::kCheckTokenId && PE_CHECK_POSITION == pe::kCheckPosition &&
                    PE_CHECK_BLOCK_TABLE == pe::kCheckBlockTable,
                "check bits");
  pe::CheckArgs a{};
  a.c = c; a.K = K; a.T = T; a.V = m->d.vocab > 0 ? m->d.vocab : INT32_MAX; a.max_blocks = max_blocks;
  a.query_lens = query_lens; a.target_ids = target_ids; a.target_pos = target_pos;
  a.num_accepted = num_accepted; a.bonus_ids = bonus_ids; a.block_table = block_table; a.error_bits = error_bits;
  PE_HIP(pe::launch_check_batch(a, stream));
  return PE_OK;
}

}  // extern "C"

namespace {
// The drafter pass behind pe_draft_forward and pe_draft_forward_noalloc;
// `timed`: launches may record kernel-timing events.
pe_status forward_impl(const pe_model* m, int32_t c, int32_t K, int32_t N, const int32_t* draft_ids,
                       const int32_t* draft_pos, const int64_t* slot_mapping, const uint8_t* is_rejected,
                       const int32_t* cu_draft, const int32_t* kv_lens, const int32_t* sample_idx,
                       const void* draft_hidden, const int32_t* block_table, int32_t max_blocks,
                       void* const* k_cache, void* const* v_cache, void* workspace, size_t workspace_bytes,
                       int32_t* draft_tokens, float* logits, float* top2_gap, hipStream_t stream, bool timed) {
  // m is read only: the handle is shared by every stream and thread
  if (!m || c <= 0 || K <= 0 || N < c * K || max_blocks <= 0) return PE_EINVAL;
  if (m->d.n_layers <= 0) return PE_EUNSUPPORTED;
  const void* ptrs[] = {draft_ids, draft_pos, slot_mapping, is_rejected, cu_draft, kv_lens,
                        sample_idx, draft_hidden, block_table, k_cache, v_cache, workspace,
                        draft_tokens};
  for (const void* p : ptrs)
    if (!p) return PE_EINVAL;
  for (int l = 0; l < m->d.n_layers; ++l)
    if (!k_cache[l] || !v_cache[l] || !aligned16(k_cache[l]) || !aligned16(v_cache[l])) return PE_EINVAL;
  if (!aligned16(draft_hidden) || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return PE_EINVAL;
  const Workspace ws = plan_workspace(m, c, K, N);
  if (workspace_bytes < ws.total) return PE_EWORKSPACE;

  const pe_model_desc& d = m->d;
  const DType t = dt(m);
  const int H = d.hidden, qd = d.n_q * d.head_dim, kvd = d.n_kv * d.head_dim, S = c * K;
  {
    // every projection's activation slice must fit the kernel's LDS budget
    const int shapes[][2] = {{N, 2 * H}, {N, H}, {N, qd}, {N, d.inter}};
    for (const auto& sh : shapes)
      if (pe::gemv_lds_bytes(sh[0], sh[1], t) > 160 * 1024) return PE_EUNSUPPORTED;
    if (pe::gemv_lds_bytes(S, H, t, pe::Epi::Argmax) > 160 * 1024) return PE_EUNSUPPORTED;
  }
  char* wb = static_cast<char*>(workspace);
  float* x = reinterpret_cast<float*>(wb + ws.x);
  void* act = wb + ws.act;
  float* qkv = reinterpret_cast<float*>(wb + ws.qkv);
  void* qrot = wb + ws.q;
  float* part = reinterpret_cast<float*>(wb + ws.attn_part);
  void* mlp = wb + ws.mlp;
  pe::Top2* top2 = reinterpret_cast<pe::Top2*>(wb + ws.top2);
  void* f = wb + ws.f;
  float* ss0 = reinterpret_cast<float*>(wb + ws.ss0);
  float* xpart = reinterpret_cast<float*>(wb + ws.part);
  const int cus = m->num_cus;

  const int ss_tiles = (H + 15) / 16;
  // rows at and past cu_draft[c] are padding (compacted layout): skipped
  const int32_t* live = cu_draft + c;
  const bool fused = fused_plan(d, N);
  const bool packed = !m->pk_layers.empty();
  // packed models split the down projection instead (the final RMSNorm adds
  // its partials for the sampled rows)
  const bool fnorm = fused && !packed && fused_final_norm(d, N, S);
  // Over more than 256 rows every projection reads a tile-major copy of its
  // weights, and the producers of the plain operands (both RMSNorms, the
  // attention merge, the SiluMul epilogue) write them tile-major in 128-row
  // groups, so that each copy into LDS reads one contiguous KiB of either.
  const bool many = fused && packed && N > 256 && m->pk_fc_tiles;
  const int og = many ? 128 : 0;
  // attention and LM head are shared by both plans
  auto attention = [&](int l) -> pe_status {
    pe::AttnArgs at{};
    at.c = c; at.N = N; at.n_q = d.n_q; at.n_kv = d.n_kv; at.d = d.head_dim;
    at.block_size = d.block_size; at.max_blocks = max_blocks; at.splits = ws.splits; at.dtype = t;
    at.q = qrot; at.pos = draft_pos; at.rejected = is_rejected; at.cu_draft = cu_draft;
    at.kv_lens = kv_lens; at.block_table = block_table; at.k_cache = k_cache[l];
    at.v_cache = v_cache[l]; at.partial = part; at.out = act; at.out_group = og;
    // the ring kernels hold two workgroups per CU
    at.fold = static_cast<int64_t>(ws.splits) * d.n_kv * c <= 2LL * cus;
    TimedScope ts(PE_KERNEL_ATTENTION, stream, timed);
    PE_HIP(pe::launch_attention(at, stream));
    return PE_OK;
  };
  auto proj = [&](pe::GemvArgs& g, pe::Epi e) -> pe_status {
    PE_HIP(pe::launch_gemv(g, e, t, cus, stream));
    return PE_OK;
  };
  // Split partials left in `part` by the last projection into x; the next
  // RMSNorm of x completes the rows (adding the residual for AddTo).
  int pend_splits = 0;
  bool pend_acc = false;
  auto into_x = [&](pe::GemvArgs& g, pe::Epi e) -> pe_status {
    // the weight-streaming kernel splits only packed weights; the tiled GEMM
    // splits when its tiles alone would leave CUs idle
    g.part = !g.ss_out && (g.pk_a || pe::proj_kernel(g.M, g.K, t) == pe::ProjKernel::Tiled) ? xpart : nullptr;
    pe_status r = proj(g, e);
    if (r != PE_OK) return r;
    pend_splits = g.splits > 1 ? g.splits : 0;
    pend_acc = e == pe::Epi::AddTo;
    return PE_OK;
  };
  // (cos, sin) of every row's rotary angles, written once by the first layer's
  // input RMSNorm and read by every layer's q/k/v epilogue
  float2* rope_tab = reinterpret_cast<float2*>(wb + ws.rope);
  auto norm_x = [&](const void* gain, bool rope_table = false) -> pe_status {
    pe::RopeTable rt{};
    if (rope_table) {
      rt.pos = draft_pos; rt.out = rope_tab; rt.half = d.head_dim / 2; rt.freq = m->freq;
    }
    PE_HIP(pe::launch_rmsnorm(t, N, H, nullptr, x, gain, d.rms_eps, act, stream, live, xpart, pend_splits, N,
                              pend_acc, og, rope_table ? &rt : nullptr));
    pend_splits = 0;
    return PE_OK;
  };
  pe_status st;

  if (fused) {
    // fc over [emb(id) ; h] gathered on the fly; epilogue emits row sums of squares
    {
      pe::GemvArgs g{};
      g.M = N; g.m_live = live; g.Nout = H; g.K = 2 * H; g.amode = pe::AMode::Gather;
      g.ids = draft_ids; g.embed = m->w.embed; g.x2 = draft_hidden;
      g.w_a = g.w_b = g.w_c = m->w.w_fc; g.n_a = H; g.n_b = 0;
      g.pk_a = packed ? m->pk_fc : nullptr;
      g.pk_tiles = many ? m->pk_fc_tiles : nullptr;
      g.y = x; g.ldy = H;
      if ((st = into_x(g, pe::Epi::Store)) != PE_OK) return st;
    }
    for (int l = 0; l < d.n_layers; ++l) {
      const pe_layer_weights& L = m->layers[l];
      const PackedLayer* P = packed ? &m->pk_layers[l] : nullptr;
      // RMSNorm as its own pass (it also completes split partials): forming it
      // inside the projection would make every workgroup re-read the fp32 rows
      if ((st = norm_x(L.ln1, l == 0)) != PE_OK) return st;
      {
        // q/k/v -> RoPE -> q operand + paged KV write
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = qd + 2 * kvd; g.K = H; g.amode = pe::AMode::Plain; g.x = act;
        g.w_a = L.wq; g.n_a = qd; g.w_b = L.wk; g.n_b = kvd; g.w_c = L.wv;
        g.pk_a = P ? P->qkv : nullptr;
        g.pk_tiles = many ? P->t_qkv : nullptr; g.x_group = og;
        g.rope.n_q = d.n_q; g.rope.n_kv = d.n_kv; g.rope.d = d.head_dim; g.rope.block_size = d.block_size;
        g.rope.slot = slot_mapping;
        g.rope.rejected = is_rejected; g.rope.q_out = qrot; g.rope.k_cache = k_cache[l];
        g.rope.v_cache = v_cache[l]; g.rope.table = rope_tab;
        if ((st = proj(g, pe::Epi::QkvRope)) != PE_OK) return st;
      }
      if ((st = attention(l)) != PE_OK) return st;
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = H; g.K = qd; g.amode = pe::AMode::Plain; g.x = act;
        g.w_a = g.w_b = g.w_c = L.wo; g.n_a = H; g.n_b = 0;
        g.pk_a = P ? P->o : nullptr;
        g.pk_tiles = many ? P->t_o : nullptr; g.x_group = og;
        g.y = x; g.ldy = H;
        if ((st = into_x(g, pe::Epi::AddTo)) != PE_OK) return st;
      }
      if ((st = norm_x(L.ln2)) != PE_OK) return st;
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = d.inter; g.K = H; g.amode = pe::AMode::Plain; g.x = act;
        g.w_a = L.w_gate; g.w_b = L.w_up; g.w_c = L.w_up; g.n_a = d.inter; g.n_b = d.inter;
        g.pk_a = P ? P->gate : nullptr; g.pk_b = P ? P->up : nullptr;
        g.pk_tiles = many ? P->t_gu : nullptr; g.x_group = og;
        g.y_op = mlp; g.ldy = d.inter; g.y_group = og;
        if ((st = proj(g, pe::Epi::SiluMul)) != PE_OK) return st;
      }
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = H; g.K = d.inter; g.amode = pe::AMode::Plain; g.x = mlp;
        g.w_a = g.w_b = g.w_c = L.w_down; g.n_a = H; g.n_b = 0;
        g.pk_a = P ? P->down : nullptr;
        g.pk_tiles = many ? P->t_down : nullptr; g.x_group = og;
        g.y = x; g.ldy = H; g.ss_out = fnorm && l == d.n_layers - 1 ? ss0 : nullptr;
        if ((st = into_x(g, pe::Epi::AddTo)) != PE_OK) return st;
      }
    }
  } else {
    PE_HIP(pe::launch_build_fc_input(t, N, H, draft_ids, m->w.embed, draft_hidden, act, stream));
    {
      pe::GemvArgs g{};
      g.M = N; g.m_live = live; g.Nout = H; g.K = 2 * H; g.amode = pe::AMode::Plain; g.x = act;
      g.w_a = m->w.w_fc; g.n_a = H; g.w_b = g.w_c = m->w.w_fc; g.n_b = 0;
      g.y = x; g.ldy = H;
      if ((st = proj(g, pe::Epi::Store)) != PE_OK) return st;
    }
    for (int l = 0; l < d.n_layers; ++l) {
      const pe_layer_weights& L = m->layers[l];
      PE_HIP(pe::launch_rmsnorm(t, N, H, nullptr, x, L.ln1, d.rms_eps, act, stream, live));
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = qd + 2 * kvd; g.K = H; g.amode = pe::AMode::Plain; g.x = act;
        g.w_a = L.wq; g.n_a = qd; g.w_b = L.wk; g.n_b = kvd; g.w_c = L.wv;
        g.y = qkv; g.ldy = qd + 2 * kvd;
        if ((st = proj(g, pe::Epi::Store)) != PE_OK) return st;
      }
      {
        pe::RopeArgs r{};
        r.N = N; r.n_q = d.n_q; r.n_kv = d.n_kv; r.d = d.head_dim; r.block_size = d.block_size;
        r.freq = m->freq; r.dtype = t; r.qkv = qkv; r.pos = draft_pos; r.slot = slot_mapping;
        r.rejected = is_rejected; r.q_out = qrot; r.k_cache = k_cache[l]; r.v_cache = v_cache[l];
        PE_HIP(pe::launch_rope_kvwrite(r, stream));
      }
      if ((st = attention(l)) != PE_OK) return st;
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = H; g.K = qd; g.amode = pe::AMode::Plain; g.x = act;
        g.w_a = g.w_b = g.w_c = L.wo; g.n_a = H; g.n_b = 0;
        g.y = x; g.ldy = H;
        if ((st = proj(g, pe::Epi::AddTo)) != PE_OK) return st;
      }
      PE_HIP(pe::launch_rmsnorm(t, N, H, nullptr, x, L.ln2, d.rms_eps, act, stream, live));
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = d.inter; g.K = H; g.amode = pe::AMode::Plain; g.x = act;
        g.w_a = L.w_gate; g.w_b = L.w_up; g.w_c = L.w_up; g.n_a = d.inter; g.n_b = d.inter;
        g.y_op = mlp; g.ldy = d.inter;
        if ((st = proj(g, pe::Epi::SiluMul)) != PE_OK) return st;
      }
      {
        pe::GemvArgs g{};
        g.M = N; g.m_live = live; g.Nout = H; g.K = d.inter; g.amode = pe::AMode::Plain; g.x = mlp;
        g.w_a = g.w_b = g.w_c = L.w_down; g.n_a = H; g.n_b = 0;
        g.y = x; g.ldy = H;
        if ((st = proj(g, pe::Epi::AddTo)) != PE_OK) return st;
      }
    }
  }
  // The LM head over many rows streams the tile-major weight copy; the final
  // RMSNorm then writes its rows tile-major too (128-row groups).
  const int lm_group = !fnorm && m->pk_lm && pe::proj_kernel(S, H, t) == pe::ProjKernel::Tiled ? 128 : 0;
  if (!fnorm)
    PE_HIP(pe::launch_rmsnorm(t, S, H, sample_idx, x, m->w.ln_f, d.rms_eps, f, stream, nullptr, xpart,
                              pend_splits, N, pend_acc, lm_group));
  // LM head + argmax over the sampled rows
  {
    pe::GemvArgs g{};
    g.M = S; g.Nout = d.vocab; g.K = H;
    if (fnorm) {
      g.amode = pe::AMode::Norm; g.xf = x; g.rows = sample_idx; g.gain = m->w.ln_f; g.ss = ss0;
      g.ss_tiles = ss_tiles; g.ss_ld = N; g.eps = d.rms_eps;
    } else {
      g.amode = pe::AMode::Plain; g.x = f;
    }
    g.w_a = g.w_b = g.w_c = m->w.w_lm; g.n_a = d.vocab; g.n_b = 0;
    g.pk_tiles = m->pk_lm;
    g.x_group = lm_group;
    g.logits = logits; g.partials = top2;
    if (pe::gemv_grid_x(S, d.vocab, pe::Epi::Argmax, t, cus, H) > ws.lm_parts) return PE_EUNSUPPORTED;
    {
      TimedScope ts(PE_KERNEL_LM_HEAD, stream, timed);
      if ((st = proj(g, pe::Epi::Argmax)) != PE_OK) return st;
    }
    PE_HIP(pe::launch_argmax_finalize(S, g.grid_x, top2, draft_tokens, top2_gap, stream));
  }
  return PE_OK;
}

// ------------------------------------------------------- allocation-free forward
// The scratch of pe_draft_forward_noalloc: a file-scope device array, one per
// GPU the library runs on, held until the process ends.  In host code its name
// is a host-side stand-in, never a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device.  No part of the
// drafter pass needs its workspace zeroed (every region is written before it
// is read within a pass), so the array is used as the previous call left it.
constexpr size_t kStaticScratch = PE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratch];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's array, looked up once per device.
pe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return PE_EHIP;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PE_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PE_OK;
}
}  // namespace

extern "C" {

pe_status pe_draft_forward(const pe_model* m, int32_t c, int32_t K, int32_t N, const int32_t* draft_ids,
                           const int32_t* draft_pos, const int64_t* slot_mapping,
                           const uint8_t* is_rejected, const int32_t* cu_draft, const int32_t* kv_lens,
                           const int32_t* sample_idx, const void* draft_hidden,
                           const int32_t* block_table, int32_t max_blocks, void* const* k_cache,
                           void* const* v_cache, void* workspace, size_t workspace_bytes,
                           int32_t* draft_tokens, float* logits, float* top2_gap, hipStream_t stream) {
  return forward_impl(m, c, K, N, draft_ids, draft_pos, slot_mapping, is_rejected, cu_draft, kv_lens, sample_idx,
                      draft_hidden, block_table, max_blocks, k_cache, v_cache, workspace, workspace_bytes,
                      draft_tokens, logits, top2_gap, stream, true);
}

pe_status pe_draft_forward_noalloc(const pe_model* m, int32_t c, int32_t K, int32_t N, const int32_t* draft_ids,
                                   const int32_t* draft_pos, const int64_t* slot_mapping,
                                   const uint8_t* is_rejected, const int32_t* cu_draft, const int32_t* kv_lens,
                                   const int32_t* sample_idx, const void* draft_hidden,
                                   const int32_t* block_table, int32_t max_blocks, void* const* k_cache,
                                   void* const* v_cache, int32_t* draft_tokens, float* logits, float* top2_gap,
                                   hipStream_t stream) {
  // the size limit is checked before any HIP call
  if (!m || c <= 0 || K <= 0 || N < c * K || m->d.n_layers <= 0) return m && m->d.n_layers <= 0 ? PE_EUNSUPPORTED
                                                                                               : PE_EINVAL;
  if (plan_workspace(m, c, K, N).total > kStaticScratch) return PE_EWORKSPACE;
  void* ws = nullptr;
  const pe_status st = scratch_of_current_device(&ws);
  if (st != PE_OK) return st;
  return forward_impl(m, c, K, N, draft_ids, draft_pos, slot_mapping, is_rejected, cu_draft, kv_lens, sample_idx,
                      draft_hidden, block_table, max_blocks, k_cache, v_cache, ws, kStaticScratch, draft_tokens,
                      logits, top2_gap, stream, false);
}

// ---------------------------------------------------------------- autoregressive baseline
namespace {
// Workspace of the autoregressive baseline: the one-token first pass over the
// T verified rows, the single-row passes, the drafter workspace they share.
struct ArWorkspace {
  size_t meta1, hid1, metak, hidk, tok, fwd, total;
  size_t fwd_bytes;
};
ArWorkspace plan_ar(const pe_model* m, int c, int T) {
  const size_t eb = m->d.dtype == PE_F32 ? 4 : 2;
  const size_t H = m->d.hidden;
  auto meta_bytes = [&](size_t rows) {
    // ids, pos (i32), slot (i64), rejected, masked (u8), hidden map (i32), cu (c+1), kv lens, sample idx
    return align_up(rows * 4) * 2 + align_up(rows * 8) + align_up(rows) * 2 + align_up(rows * 4) +
           align_up(size_t(c + 1) * 4) + align_up(size_t(c) * 4) * 2;
  };
  ArWorkspace w{};
  size_t off = 0;
  w.meta1 = off; off += meta_bytes(T);
  w.hid1 = off;  off += align_up(size_t(T) * H * eb);
  w.metak = off; off += meta_bytes(c);
  w.hidk = off;  off += align_up(size_t(c) * H * eb);
  w.tok = off;   off += align_up(size_t(c) * 4);
  const size_t f1 = plan_workspace(m, c, 1, T).total, fk = plan_workspace(m, c, 1, c).total;
  w.fwd_bytes = f1 > fk ? f1 : fk;
  w.fwd = off;   off += w.fwd_bytes;
  w.total = off;
  return w;
}
struct MetaView {
  int32_t *ids, *pos;
  int64_t* slot;
  uint8_t *rej, *msk;
  int32_t *hmap, *cu, *kvl, *sidx;
};
MetaView carve_meta(char* base, size_t rows, int c) {
  MetaView v{};
  size_t off = 0;
  v.ids = reinterpret_cast<int32_t*>(base + off);  off += align_up(rows * 4);
  v.pos = reinterpret_cast<int32_t*>(base + off);  off += align_up(rows * 4);
  v.slot = reinterpret_cast<int64_t*>(base + off); off += align_up(rows * 8);
  v.rej = reinterpret_cast<uint8_t*>(base + off);  off += align_up(rows);
  v.msk = reinterpret_cast<uint8_t*>(base + off);  off += align_up(rows);
  v.hmap = reinterpret_cast<int32_t*>(base + off); off += align_up(rows * 4);
  v.cu = reinterpret_cast<int32_t*>(base + off);   off += align_up(size_t(c + 1) * 4);
  v.kvl = reinterpret_cast<int32_t*>(base + off);  off += align_up(size_t(c) * 4);
  v.sidx = reinterpret_cast<int32_t*>(base + off);
  return v;
}
}  // namespace

size_t pe_autoregressive_workspace_bytes(const pe_model* m, int32_t c, int32_t K, int32_t T) {
  if (!m || c <= 0 || K <= 0 || T < c) return 0;
  return plan_ar(m, c, T).total;
}

pe_status pe_draft_autoregressive(const pe_model* m, int32_t c, int32_t K, int32_t T,
                                  const int32_t* query_lens, const int32_t* target_ids,
                                  const int32_t* target_pos, const int32_t* num_accepted,
                                  const int32_t* bonus_ids, const void* target_hidden,
                                  const int32_t* block_table, int32_t max_blocks, void* const* k_cache,
                                  void* const* v_cache, void* workspace, size_t workspace_bytes,
                                  int32_t* draft_tokens, float* logits, void* fed_hidden, hipStream_t stream) {
  if (!m || c <= 0 || K <= 0 || T < c || max_blocks <= 0 || !workspace || !draft_tokens) return PE_EINVAL;
  if (m->d.n_layers <= 0) return PE_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return PE_EINVAL;
  if (fed_hidden && !aligned16(fed_hidden)) return PE_EINVAL;
  const ArWorkspace ws = plan_ar(m, c, T);
  if (workspace_bytes < ws.total) return PE_EWORKSPACE;
  char* wb = static_cast<char*>(workspace);
  const MetaView m1 = carve_meta(wb + ws.meta1, size_t(T), c);
  const MetaView mk = carve_meta(wb + ws.metak, size_t(c), c);
  int32_t* tok = reinterpret_cast<int32_t*>(wb + ws.tok);
  void* fwd = wb + ws.fwd;
  pe_status st;
  // pass 1: the verified rows with the bonus token, no MASK rows (one token)
  if ((st = pe_prepare_draft_batch(m, c, 1, T, query_lens, target_ids, target_pos, num_accepted, bonus_ids,
                                   target_hidden, block_table, max_blocks, m1.ids, m1.pos, m1.slot, m1.rej,
                                   m1.msk, m1.hmap, m1.cu, m1.kvl, m1.sidx, wb + ws.hid1, stream)) != PE_OK)
    return st;
  if ((st = pe_draft_forward(m, c, 1, T, m1.ids, m1.pos, m1.slot, m1.rej, m1.cu, m1.kvl, m1.sidx,
                             wb + ws.hid1, block_table, max_blocks, k_cache, v_cache, fwd, ws.fwd_bytes, tok,
                             logits, nullptr, stream)) != PE_OK)
    return st;
  // passes 2..K: one row per sequence fed with its own previous token and
  // final residual (the drafter workspace's residual region sits at offset 0)
  const size_t hid_bytes = size_t(c) * m->d.hidden * (m->d.dtype == PE_F32 ? 4 : 2);
  for (int k = 1; k <= K; ++k) {
    // hidden rows of pass k: the caller's buffer when given, else scratch
    void* hid = fed_hidden && k < K ? static_cast<char*>(fed_hidden) + (k - 1) * hid_bytes : wb + ws.hidk;
    pe::ArStepArgs a{};
    a.c = c; a.K = K; a.k = k; a.H = m->d.hidden; a.max_blocks = max_blocks; a.last = k == K;
    a.dtype = dt(m); a.prev_tokens = tok; a.x = reinterpret_cast<const float*>(fwd);
    a.prev_sample_idx = k == 1 ? m1.sidx : nullptr; a.base_kv_lens = m1.kvl; a.block_table = block_table;
    a.draft_tokens = draft_tokens; a.ids = mk.ids; a.pos = mk.pos; a.slot = mk.slot; a.rejected = mk.rej;
    a.cu_draft = mk.cu; a.kv_lens = mk.kvl; a.sample_idx = mk.sidx; a.hidden = hid;
    PE_HIP(pe::launch_ar_step(a, stream));
    if (k == K) break;
    if ((st = pe_draft_forward(m, c, 1, c, mk.ids, mk.pos, mk.slot, mk.rej, mk.cu, mk.kvl, mk.sidx,
                               hid, block_table, max_blocks, k_cache, v_cache, fwd, ws.fwd_bytes, tok,
                               logits ? logits + static_cast<size_t>(k) * c * m->d.vocab : nullptr, nullptr,
                               stream)) != PE_OK)
      return st;
  }
  return PE_OK;
}

pe_status pe_next_verified_batch(int32_t c, int32_t K, const int32_t* kv_lens, const int32_t* bonus_ids,
                                 const int32_t* draft_tokens, const int32_t* num_accepted_next,
                                 const int32_t* bonus_next, int32_t* query_lens_out, int32_t* target_ids_out,
                                 int32_t* target_pos_out, int32_t* num_accepted_out, int32_t* bonus_ids_out,
                                 hipStream_t stream) {
  if (c <= 0 || K <= 0) return PE_EINVAL;
  const void* ptrs[] = {kv_lens, bonus_ids, draft_tokens, num_accepted_next, bonus_next, query_lens_out,
                        target_ids_out, target_pos_out, num_accepted_out, bonus_ids_out};
  for (const void* p : ptrs)
    if (!p) return PE_EINVAL;
  PE_HIP(pe::launch_next_batch(c, K, kv_lens, bonus_ids, draft_tokens, num_accepted_next, bonus_next,
                               query_lens_out, target_ids_out, target_pos_out, num_accepted_out, bonus_ids_out,
                               stream));
  return PE_OK;
}

pe_status pe_accept(int32_t c, int32_t K, const int32_t* draft, const int32_t* target, int32_t* acc,
                    int32_t* bonus, hipStream_t stream) {
  if (c <= 0 || K <= 0 || !draft || !target || !acc || !bonus) return PE_EINVAL;
  PE_HIP(pe::launch_accept(c, K, draft, target, acc, bonus, stream));
  return PE_OK;
}

pe_status pe_timing_enable(pe_kernel_class k, int32_t enable) {
  if (k < PE_KERNEL_LM_HEAD || k > PE_KERNEL_ATTENTION) return PE_EINVAL;
  std::lock_guard<std::mutex> g(g_timing_mu);
  g_timing[k].enabled.store(enable != 0, std::memory_order_relaxed);
  g_timing[k].used = 0;
  return PE_OK;
}

pe_status pe_timing_read(pe_kernel_class k, double* total_ms, int64_t* launches, float* per_launch_ms,
                         int64_t capacity) {
  if (!total_ms || !launches || k < PE_KERNEL_LM_HEAD || k > PE_KERNEL_ATTENTION) return PE_EINVAL;
  if (per_launch_ms && capacity < 0) return PE_EINVAL;
  std::lock_guard<std::mutex> g(g_timing_mu);
  Timing& t = g_timing[k];
  double sum = 0.0;
  for (size_t i = 0; i < t.used; ++i) {
    PE_HIP(hipEventSynchronize(t.events[i].second));
    float ms = 0.f;
    PE_HIP(hipEventElapsedTime(&ms, t.events[i].first, t.events[i].second));
    if (per_launch_ms && static_cast<int64_t>(i) < capacity) per_launch_ms[i] = ms;
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int64_t>(t.used);
  return PE_OK;
}

}  // extern "C"
