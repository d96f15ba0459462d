// C ABI of libfixedm: argument validation, descriptor/state bookkeeping and kernel dispatch.
// Every host-checkable error is reported before anything is enqueued.
//
// Sources (page title, section):
//   [FM] "feat(attention): fixed-m splash attention kernel with dynamic bounds and safety
//        fallbacks": Summary (C(N), W(N), gate), commit message (metadata contracts raise
//        at entry; fp16/fp8 rejected).
//   [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention":
//        Interface table (softmax_scale defaults to 1/sqrt(d)), Overview ring figure (step 0
//        initialises, later steps add), Best practices (no selector for the only path).
#include <math.h>
#include <string.h>

#include "fixedm_internal.h"

using namespace fixedm;

namespace {

constexpr double kLog2e = 1.4426950408889634;  // log2(e), fp64

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int32_t ceil_log2_i64(int64_t n) {
  int32_t L = 0;
  while (L < 63 && ((int64_t)1 << L) < n) ++L;
  return L;
}

fixedm_status check_problem(const fixedm_problem* p) {
  if (p == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (p->abi_version != FIXEDM_ABI_VERSION) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (p->dtype != FIXEDM_BF16 && p->dtype != FIXEDM_F32) return FIXEDM_ERR_UNSUPPORTED_DTYPE;
  if (p->batch < 1 || p->heads < 1 || p->sq < 1 || p->sk_total < 1 || p->head_dim < 1)
    return FIXEDM_ERR_INVALID_ARGUMENT;
  if (p->center < FIXEDM_CENTER_NONE || p->center > FIXEDM_CENTER_COMPUTE)
    return FIXEDM_ERR_INVALID_ARGUMENT;
  if (p->shift != FIXEDM_SHIFT_BLOCK && p->shift != FIXEDM_SHIFT_ROW) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale >= 0.0f) || !isfinite(p->softmax_scale)) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (p->dtype == FIXEDM_BF16 && p->head_dim != 128) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  if (p->dtype == FIXEDM_F32 && p->head_dim != 64 && p->head_dim != 128) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  if (p->q_block < 64 || p->q_block % 64 != 0) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  // grid limits of the kernels (y dimension = B*H; 32-bit row indices)
  if (p->batch > 65535 || p->heads > 65535 || p->batch * p->heads > 65535) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  if (p->sq > (int64_t)1 << 30 || p->sk_total > kMaxKeys) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  // bf16: the key tiles of one launch are counted in 32 bits
  if (p->dtype == FIXEDM_BF16 && p->sk_total > kMaxKeysBf16) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  const int64_t n_qtiles = (p->sq + kQTile - 1) / kQTile;
  if (p->batch * p->heads * n_qtiles > ((int64_t)1 << 31) - 1) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  return FIXEDM_OK;
}

float resolved_scale(const fixedm_problem& p) {
  if (p.softmax_scale > 0.0f) return p.softmax_scale;
  return (float)(1.0 / sqrt((double)p.head_dim));
}

fixedm_status check_tensor(const fixedm_problem& p, const fixedm_tensor& t) {
  if (t.ptr == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)t.ptr & 15) != 0) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  const int64_t vec = p.dtype == FIXEDM_BF16 ? 8 : 4;  // elements per 16 bytes
  if (t.stride_b < 0 || t.stride_s < 0 || t.stride_h < 0) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  if (t.stride_b % vec || t.stride_s % vec || t.stride_h % vec) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  // The bf16 attention kernel's K/V loads take a row's byte offset within a 32-row tile as
  // an unsigned 32-bit lane offset (31 rows x stride_s x 2 bytes + 240 must stay below 2^32).
  if (p.dtype == FIXEDM_BF16 && t.stride_s > kMaxRowStrideBf16) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  return FIXEDM_OK;
}

fixedm_status check_out_tensor(const fixedm_problem& p, const fixedm_tensor& t, int32_t dt) {
  if (t.ptr == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)t.ptr & 15) != 0) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  const int64_t vec = dt == FIXEDM_BF16 ? 4 : 4;  // 4 elements per store (8 or 16 bytes)
  if (t.stride_b < 0 || t.stride_s < 0 || t.stride_h < 0) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  if (t.stride_b % vec || t.stride_s % vec || t.stride_h % vec) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  (void)p;
  return FIXEDM_OK;
}

fixedm_status check_chunks(const fixedm_problem& p, const fixedm_tensor* kc, const fixedm_tensor* vc,
                           const int64_t* len, int32_t n, int64_t* total) {
  if (n < 1 || kc == nullptr || vc == nullptr || len == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  int64_t s = 0;
  for (int32_t c = 0; c < n; ++c) {
    // each length and the running sum stay within the key limit, so the sum cannot wrap
    if (len[c] < 0 || len[c] > kMaxKeys) return FIXEDM_ERR_INVALID_ARGUMENT;
    if (len[c] == 0) continue;
    fixedm_status st = check_tensor(p, kc[c]);
    if (st != FIXEDM_OK) return st;
    st = check_tensor(p, vc[c]);
    if (st != FIXEDM_OK) return st;
    s += len[c];
    if (s > kMaxKeys) return FIXEDM_ERR_INVALID_ARGUMENT;
  }
  *total = s;
  return FIXEDM_OK;
}

uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const unsigned char* c = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= c[i];
    h *= 1099511628211ull;
  }
  return h;
}

uint64_t descriptor_token(const fixedm_bounds_t& b) {
  uint64_t h = 14695981039346656037ull;
  const fixedm_problem& p = b.p;
  h = fnv1a(h, &p.abi_version, sizeof p.abi_version);
  h = fnv1a(h, &p.dtype, sizeof p.dtype);
  h = fnv1a(h, &p.batch, sizeof p.batch);
  h = fnv1a(h, &p.heads, sizeof p.heads);
  h = fnv1a(h, &p.head_dim, sizeof p.head_dim);
  h = fnv1a(h, &p.sq, sizeof p.sq);
  h = fnv1a(h, &p.sk_total, sizeof p.sk_total);
  h = fnv1a(h, &p.q_block, sizeof p.q_block);
  h = fnv1a(h, &p.softmax_scale, sizeof p.softmax_scale);
  h = fnv1a(h, &p.center, sizeof p.center);
  h = fnv1a(h, &p.shift, sizeof p.shift);
  h = fnv1a(h, &b.log2_n, sizeof b.log2_n);
  h = fnv1a(h, &b.C, sizeof b.C);
  h = fnv1a(h, &b.W, sizeof b.W);
  h = fnv1a(h, &b.gate, sizeof b.gate);
  h = fnv1a(h, &b.n_qblocks, sizeof b.n_qblocks);
  h = fnv1a(h, &b.alpha, sizeof b.alpha);
  h = fnv1a(h, &b.dev, sizeof b.dev);
  return h | 1ull;  // never 0, so a zeroed run state never matches
}

fixedm_status check_descriptor(const fixedm_bounds_t* b) {
  if (b == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (b->dev == nullptr || b->token == 0) return FIXEDM_ERR_BOUNDS_MISMATCH;
  if (check_problem(&b->p) != FIXEDM_OK) return FIXEDM_ERR_BOUNDS_MISMATCH;
  if (descriptor_token(*b) != b->token) return FIXEDM_ERR_BOUNDS_MISMATCH;
  return FIXEDM_OK;
}

ChunkDesc make_chunk(const fixedm_tensor& k, const fixedm_tensor& v, int64_t len, int64_t start) {
  ChunkDesc c;
  c.k = k.ptr;
  c.v = v.ptr;
  c.k_sb = k.stride_b; c.k_ss = k.stride_s; c.k_sh = k.stride_h;
  c.v_sb = v.stride_b; c.v_ss = v.stride_s; c.v_sh = v.stride_h;
  c.len = len;
  c.start = start;
  return c;
}

}  // namespace

namespace fixedm {

bool bounds_layout(const fixedm_problem& p, BoundsLayout* out) {
  if (check_problem(&p) != FIXEDM_OK) return false;
  const size_t nqb = (size_t)((p.sq + p.q_block - 1) / p.q_block);
  const size_t bh = (size_t)(p.batch * p.heads);
  size_t off = 0;
  out->m = off; off = align256(off + bh * nqb * 4);
  out->elig = off; off = align256(off + bh * nqb);
  out->u = off; off = align256(off + bh * nqb * 8);
  out->q2 = off; off = align256(off + bh * nqb * 8);
  out->k2 = off; off = align256(off + bh * 8);
  out->k_mean = off; off = align256(off + bh * (size_t)p.head_dim * 4);
  out->v_bad = off; off = align256(off + 4);
  const size_t rows = p.shift == FIXEDM_SHIFT_ROW ? bh * (size_t)p.sq : 0;
  out->m_row = off; off = align256(off + rows * 4);
  out->q2_row = off; off = align256(off + rows * 8);
  out->u_row = off; off = align256(off + rows * 8);
  out->scratch = off;
  off += bounds_scratch(p).total;           // key-mean partial sums and flags (COMPUTE only)
  out->total = off;
  return true;
}

bool workspace_layout(const fixedm_problem& p, WorkspaceLayout* out) {
  if (check_problem(&p) != FIXEDM_OK) return false;
  out->n_qtiles = (p.sq + kQTile - 1) / kQTile;
  out->sq_pad = out->n_qtiles * kQTile;
  const size_t rows = (size_t)(p.batch * p.heads * out->sq_pad);
  size_t off = 0;
  out->acc = off; off = align256(off + rows * (size_t)p.head_dim * 4);
  out->l = off; off = align256(off + rows * 4);
  out->r = off; off = align256(off + rows * 4);
  out->acc_x = out->l_x = out->r_x = off;
  if (p.dtype == FIXEDM_BF16) {
    const int64_t tiles = p.batch * p.heads * out->n_qtiles;
    const size_t xt = (size_t)(kMaxParts - 1) * (size_t)(tiles < kMaxSplitTail ? tiles : kMaxSplitTail);
    out->acc_x = off; off = align256(off + xt * kQTile * (size_t)p.head_dim * 4);
    out->l_x = off; off = align256(off + xt * kQTile * 4);
    out->r_x = off; off = align256(off + xt * kQTile * 4);
  }
  out->queue = off;
  if (p.dtype == FIXEDM_BF16) off = align256(off + 16 * sizeof(unsigned long long));
  out->slow_list = off;
  if (p.dtype == FIXEDM_BF16) off = align256(off + (size_t)(p.batch * p.heads * out->n_qtiles) * 4);
  out->ptable = off;
  if (p.dtype == FIXEDM_BF16)
    off = align256(off + (size_t)(p.batch * p.heads) * kPieceLists * kPieceSlots * kPieceWords * 4);
  out->total = off;
  return true;
}

int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

}  // namespace fixedm

extern "C" {

const char* fixedm_status_string(fixedm_status s) {
  switch (s) {
    case FIXEDM_OK: return "FIXEDM_OK";
    case FIXEDM_ERR_INVALID_ARGUMENT: return "FIXEDM_ERR_INVALID_ARGUMENT";
    case FIXEDM_ERR_UNSUPPORTED_DTYPE: return "FIXEDM_ERR_UNSUPPORTED_DTYPE";
    case FIXEDM_ERR_UNSUPPORTED_SHAPE: return "FIXEDM_ERR_UNSUPPORTED_SHAPE";
    case FIXEDM_ERR_BOUNDS_MISMATCH: return "FIXEDM_ERR_BOUNDS_MISMATCH";
    case FIXEDM_ERR_STATE: return "FIXEDM_ERR_STATE";
    case FIXEDM_ERR_HIP: return "FIXEDM_ERR_HIP";
  }
  return "FIXEDM_UNKNOWN_STATUS";
}

fixedm_status fixedm_constants(int64_t n, int32_t* log2_n, int32_t* C, int32_t* W, int32_t* gate) {
  if (n < 1) return FIXEDM_ERR_INVALID_ARGUMENT;
  const int32_t L = ceil_log2_i64(n);
  const int32_t c = 127 - L - 8;  // ceil(log2 Vmax) = 8 for Vmax = 256
  const int32_t w = c + 125;
  if (log2_n) *log2_n = L;
  if (C) *C = c;
  if (W) *W = w;
  if (gate) *gate = w >= 0 ? w / 2 : -((-w + 1) / 2);  // floor(w / 2)
  return FIXEDM_OK;
}

size_t fixedm_bounds_bytes(const fixedm_problem* p) {
  BoundsLayout l;
  if (p == nullptr || !bounds_layout(*p, &l)) return 0;
  return l.total;
}

fixedm_status fixedm_bounds_layout(const fixedm_problem* p, fixedm_bounds_layout_t* out) {
  const fixedm_status st = check_problem(p);
  if (st != FIXEDM_OK) return st;
  if (out == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  BoundsLayout l;
  bounds_layout(*p, &l);
  out->m = l.m; out->elig = l.elig; out->u = l.u; out->q2 = l.q2; out->k2 = l.k2;
  out->k_mean = l.k_mean; out->v_bad = l.v_bad; out->m_row = l.m_row; out->q2_row = l.q2_row;
  out->u_row = l.u_row; out->scratch = l.scratch; out->total = l.total;
  return FIXEDM_OK;
}

size_t fixedm_workspace_bytes(const fixedm_problem* p) {
  WorkspaceLayout w;
  if (p == nullptr || !workspace_layout(*p, &w)) return 0;
  return w.total;
}

}  // extern "C"

namespace {

// fixedm_bounds and fixedm_bounds_static: the checks, the descriptor and the launches.
// bounds_dev holds the outputs (need_bytes of it checked); the scratch of COMPUTE centring
// lies at scratch_base with the given layout, or (scratch_base null) in the static array,
// whose address is looked up only once every host-checkable error has been ruled out.
fixedm_status bounds_impl(const fixedm_problem* p, fixedm_tensor q, const fixedm_tensor* k_chunks,
                          const fixedm_tensor* v_chunks, const int64_t* chunk_len, int32_t n_chunks,
                          const float* k_mean_in, void* bounds_dev, size_t bounds_dev_bytes,
                          size_t need_bytes, char* scratch_base, const BoundsScratch& sc,
                          fixedm_bounds_t* out, void* stream) {
  fixedm_status st = FIXEDM_OK;
  if (out == nullptr || bounds_dev == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (bounds_dev_bytes < need_bytes) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)bounds_dev & 255) != 0) return FIXEDM_ERR_INVALID_ARGUMENT;
  if ((st = check_tensor(*p, q)) != FIXEDM_OK) return st;
  if (n_chunks > kMaxBoundsChunks) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  int64_t total = 0;
  if ((st = check_chunks(*p, k_chunks, v_chunks, chunk_len, n_chunks, &total)) != FIXEDM_OK) return st;
  if (total != p->sk_total) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (p->center == FIXEDM_CENTER_SUPPLIED) {
    if (k_mean_in == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)k_mean_in & 3) != 0) return FIXEDM_ERR_INVALID_ARGUMENT;
  }
  if (scratch_base == nullptr && sc.total > 0) {
    scratch_base = static_cast<char*>(static_scratch());
    if (scratch_base == nullptr) return FIXEDM_ERR_HIP;
  }

  fixedm_bounds_t d;
  memset(&d, 0, sizeof d);
  d.p = *p;
  d.p.softmax_scale = resolved_scale(*p);
  fixedm_constants(p->sk_total, &d.log2_n, &d.C, &d.W, &d.gate);
  d.n_qblocks = (p->sq + p->q_block - 1) / p->q_block;
  const double alpha64 = (double)d.p.softmax_scale * kLog2e;
  d.alpha = (float)alpha64;
  d.dev = bounds_dev;
  d.token = descriptor_token(d);

  BoundsLayout lay;
  bounds_layout(*p, &lay);
  char* base = static_cast<char*>(bounds_dev);
  BoundsArgs a;
  memset(&a, 0, sizeof a);
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_ss = q.stride_s; a.q_sh = q.stride_h;
  int32_t nc = 0;
  int64_t start = 0;
  for (int32_t c = 0; c < n_chunks; ++c) {
    if (chunk_len[c] == 0) continue;
    a.ch[nc++] = make_chunk(k_chunks[c], v_chunks[c], chunk_len[c], start);
    start += chunk_len[c];
  }
  a.n_chunks = nc;
  a.dtype = p->dtype;
  a.B = (int32_t)p->batch; a.H = (int32_t)p->heads; a.D = (int32_t)p->head_dim;
  a.Sq = p->sq; a.N = p->sk_total; a.q_block = p->q_block; a.nqb = d.n_qblocks;
  a.center = p->center;
  a.k_mean_in = k_mean_in;
  a.alpha64 = alpha64;
  a.C = d.C; a.gate = d.gate;
  a.m = reinterpret_cast<int32_t*>(base + lay.m);
  a.elig = reinterpret_cast<uint8_t*>(base + lay.elig);
  a.u = reinterpret_cast<double*>(base + lay.u);
  a.q2 = reinterpret_cast<unsigned long long*>(base + lay.q2);
  a.k2 = reinterpret_cast<unsigned long long*>(base + lay.k2);
  a.k_mean = reinterpret_cast<float*>(base + lay.k_mean);
  a.v_bad = reinterpret_cast<int32_t*>(base + lay.v_bad);
  a.kpart = reinterpret_cast<double*>(scratch_base + sc.kpart);
  a.kflag = reinterpret_cast<uint8_t*>(scratch_base + sc.kflag);
  a.kslabs = sc.slabs;
  if (p->shift == FIXEDM_SHIFT_ROW) {
    a.m_row = reinterpret_cast<int32_t*>(base + lay.m_row);
    a.q2_row = reinterpret_cast<double*>(base + lay.q2_row);
    a.u_row = reinterpret_cast<double*>(base + lay.u_row);
  }
  if (launch_bounds(a, static_cast<hipStream_t>(stream)) != hipSuccess) return FIXEDM_ERR_HIP;
  *out = d;
  return FIXEDM_OK;
}

}  // namespace

extern "C" {

fixedm_status fixedm_bounds(const fixedm_problem* p, fixedm_tensor q, const fixedm_tensor* k_chunks,
                            const fixedm_tensor* v_chunks, const int64_t* chunk_len, int32_t n_chunks,
                            const float* k_mean_in, void* bounds_dev, size_t bounds_dev_bytes,
                            fixedm_bounds_t* out, void* stream) {
  const fixedm_status st = check_problem(p);
  if (st != FIXEDM_OK) return st;
  BoundsLayout lay;
  bounds_layout(*p, &lay);
  return bounds_impl(p, q, k_chunks, v_chunks, chunk_len, n_chunks, k_mean_in, bounds_dev, bounds_dev_bytes,
                     lay.total, static_cast<char*>(bounds_dev) + lay.scratch, bounds_scratch(*p), out, stream);
}

fixedm_status fixedm_bounds_static(const fixedm_problem* p, fixedm_tensor q, const fixedm_tensor* k_chunks,
                                   const fixedm_tensor* v_chunks, const int64_t* chunk_len, int32_t n_chunks,
                                   const float* k_mean_in, void* bounds_dev, size_t bounds_dev_bytes,
                                   fixedm_bounds_t* out, void* stream) {
  const fixedm_status st = check_problem(p);
  if (st != FIXEDM_OK) return st;
  BoundsLayout lay;
  bounds_layout(*p, &lay);
  // as few key slabs as the static array needs: its size bounds the partial sums
  const size_t el = (size_t)(p->batch * p->heads) * (size_t)p->head_dim;
  if (kStaticScratchBytes < el * 9 + 512) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  const BoundsScratch sc = bounds_scratch(*p, (int64_t)((kStaticScratchBytes - 512) / (el * 9)));
  if (sc.total > kStaticScratchBytes) return FIXEDM_ERR_UNSUPPORTED_SHAPE;
  return bounds_impl(p, q, k_chunks, v_chunks, chunk_len, n_chunks, k_mean_in, bounds_dev, bounds_dev_bytes,
                     lay.scratch, nullptr, sc, out, stream);
}

fixedm_status fixedm_run_init(const fixedm_bounds_t* bounds, fixedm_run_t* run) {
  const fixedm_status st = check_descriptor(bounds);
  if (st != FIXEDM_OK) return st;
  if (run == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  run->token = bounds->token;
  run->kv_visited = 0;
  run->calls = 0;
  run->finalized = 0;
  return FIXEDM_OK;
}

}  // extern "C"

namespace {

// Shared checks of the attention entry points; fills *total with the keys of the call.
fixedm_status check_attn_call(const fixedm_bounds_t* bounds, const fixedm_run_t* run, fixedm_tensor q,
                              const fixedm_tensor* k_chunks, const fixedm_tensor* v_chunks,
                              const int64_t* chunk_len, int32_t n_chunks, const void* workspace,
                              size_t workspace_bytes, int64_t* total, bool allow_none = false) {
  fixedm_status st = check_descriptor(bounds);
  if (st != FIXEDM_OK) return st;
  if (run == nullptr || workspace == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fixedm_workspace_bytes(&bounds->p)) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (run->token != bounds->token) return FIXEDM_ERR_BOUNDS_MISMATCH;
  if (((uintptr_t)workspace & 255) != 0) return FIXEDM_ERR_INVALID_ARGUMENT;
  const fixedm_problem& p = bounds->p;
  if ((st = check_tensor(p, q)) != FIXEDM_OK) return st;
  *total = 0;
  if (!(allow_none && n_chunks == 0) &&
      (st = check_chunks(p, k_chunks, v_chunks, chunk_len, n_chunks, total)) != FIXEDM_OK)
    return st;
  if (run->finalized != 0) return FIXEDM_ERR_STATE;
  if (run->kv_visited < 0 || run->kv_visited > p.sk_total || run->kv_visited + *total > p.sk_total)
    return FIXEDM_ERR_STATE;
  return FIXEDM_OK;
}

fixedm_status check_out_call(const fixedm_problem& p, fixedm_tensor out, int32_t out_dtype, const float* lse) {
  if (out_dtype != FIXEDM_BF16 && out_dtype != FIXEDM_F32) return FIXEDM_ERR_UNSUPPORTED_DTYPE;
  const fixedm_status st = check_out_tensor(p, out, out_dtype);
  if (st != FIXEDM_OK) return st;
  if (lse != nullptr && ((uintptr_t)lse & 3) != 0) return FIXEDM_ERR_INVALID_ARGUMENT;
  return FIXEDM_OK;
}

SplitPlan plan_of(const fixedm_problem& p, const WorkspaceLayout& wl) {
  const int64_t tiles = p.batch * p.heads * wl.n_qtiles;
  return p.dtype == FIXEDM_BF16 ? split_plan(tiles, device_cus(), (p.sk_total + 31) / 32)
                                : SplitPlan{(int32_t)tiles, 1};
}

AttnArgs attn_args(const fixedm_bounds_t* bounds, fixedm_tensor q, void* workspace) {
  const fixedm_problem& p = bounds->p;
  BoundsLayout lay;
  bounds_layout(p, &lay);
  WorkspaceLayout wl;
  workspace_layout(p, &wl);
  const char* bbase = static_cast<const char*>(bounds->dev);
  char* wbase = static_cast<char*>(workspace);
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_ss = q.stride_s; a.q_sh = q.stride_h;
  a.B = (int32_t)p.batch; a.H = (int32_t)p.heads; a.D = (int32_t)p.head_dim;
  a.Sq = (int32_t)p.sq; a.n_qtiles = (int32_t)wl.n_qtiles; a.sq_pad = (int32_t)wl.sq_pad;
  a.q_block = (int32_t)p.q_block; a.nqb = (int32_t)bounds->n_qblocks;
  a.m = reinterpret_cast<const int32_t*>(bbase + lay.m);
  a.m_row = p.shift == FIXEDM_SHIFT_ROW ? reinterpret_cast<const int32_t*>(bbase + lay.m_row) : nullptr;
  a.elig = reinterpret_cast<const uint8_t*>(bbase + lay.elig);
  a.u = reinterpret_cast<const double*>(bbase + lay.u);
  a.k_mean = reinterpret_cast<const float*>(bbase + lay.k_mean);
  a.v_bad = reinterpret_cast<const int32_t*>(bbase + lay.v_bad);
  a.log2_n = bounds->log2_n;
  a.alpha = bounds->alpha;
  a.alpha64 = (double)p.softmax_scale * kLog2e;
  a.acc = reinterpret_cast<float*>(wbase + wl.acc);
  a.l = reinterpret_cast<float*>(wbase + wl.l);
  a.r = reinterpret_cast<float*>(wbase + wl.r);
  a.acc_x = reinterpret_cast<float*>(wbase + wl.acc_x);
  a.l_x = reinterpret_cast<float*>(wbase + wl.l_x);
  a.r_x = reinterpret_cast<float*>(wbase + wl.r_x);
  a.queue = reinterpret_cast<unsigned long long*>(wbase + wl.queue);
  a.slow_list = reinterpret_cast<int32_t*>(wbase + wl.slow_list);
  a.ptable = reinterpret_cast<uint32_t*>(wbase + wl.ptable);
  const SplitPlan sp = plan_of(p, wl);
  a.n_whole = sp.n_whole;
  a.parts = sp.parts;
  return a;
}

FinalizeArgs finalize_args(const fixedm_problem& p, const void* workspace, fixedm_tensor out, int32_t out_dtype,
                           float* lse) {
  WorkspaceLayout wl;
  workspace_layout(p, &wl);
  const char* wbase = static_cast<const char*>(workspace);
  FinalizeArgs a;
  memset(&a, 0, sizeof a);
  a.acc = reinterpret_cast<const float*>(wbase + wl.acc);
  a.l = reinterpret_cast<const float*>(wbase + wl.l);
  a.r = reinterpret_cast<const float*>(wbase + wl.r);
  a.out = const_cast<void*>(out.ptr);
  a.o_sb = out.stride_b; a.o_ss = out.stride_s; a.o_sh = out.stride_h;
  a.out_dtype = out_dtype;
  a.lse = lse;
  a.B = (int32_t)p.batch; a.H = (int32_t)p.heads; a.D = (int32_t)p.head_dim;
  a.Sq = (int32_t)p.sq; a.n_qtiles = (int32_t)wl.n_qtiles; a.sq_pad = (int32_t)wl.sq_pad;
  a.reg_layout = p.dtype == FIXEDM_BF16 ? 1 : 0;
  const SplitPlan sp = plan_of(p, wl);
  a.n_whole = sp.n_whole;
  a.parts = sp.parts;
  a.tile_begin = 0;
  a.acc_x = reinterpret_cast<const float*>(wbase + wl.acc_x);
  a.l_x = reinterpret_cast<const float*>(wbase + wl.l_x);
  a.r_x = reinterpret_cast<const float*>(wbase + wl.r_x);
  return a;
}

// Enqueues the attention launches of one call: up to kMaxChunksPerLaunch non-empty chunks per
// launch, each launch folding its chunks into registers and then into the workspace.  With
// `fin` (bf16 only) the last launch completes the run and writes O itself (fin->... fields).
fixedm_status enqueue_attn(AttnArgs a, const fixedm_problem& p, const fixedm_tensor* k_chunks,
                           const fixedm_tensor* v_chunks, const int64_t* chunk_len, int32_t n_chunks,
                           int64_t visited, const AttnArgs* fin, hipStream_t s) {
  int32_t c = 0;
  while (c < n_chunks) {
    a.n_chunks = 0;
    a.call_len = 0;
    a.call_tiles = 0;
    while (c < n_chunks && a.n_chunks < kMaxChunksPerLaunch) {
      if (chunk_len[c] > 0) {
        a.ch[a.n_chunks++] = make_chunk(k_chunks[c], v_chunks[c], chunk_len[c], a.call_len);
        a.call_len += chunk_len[c];
        a.call_tiles += (chunk_len[c] + 31) / 32;
      }
      ++c;
    }
    while (c < n_chunks && chunk_len[c] == 0) ++c;   // trailing empty chunks end the call here
    if (a.n_chunks == 0) break;
    a.accumulate = visited > 0 ? 1 : 0;
    if (fin != nullptr && c == n_chunks) {
      a.final_out = 1;
      a.out_dtype = fin->out_dtype;
      a.out = fin->out;
      a.o_sb = fin->o_sb; a.o_ss = fin->o_ss; a.o_sh = fin->o_sh;
      a.lse = fin->lse;
    }
    const hipError_t e = p.dtype == FIXEDM_BF16 ? launch_attn_bf16(a, s) : launch_attn_f32(a, s);
    if (e != hipSuccess) return FIXEDM_ERR_HIP;
    visited += a.call_len;
  }
  return FIXEDM_OK;
}

}  // namespace

extern "C" {

fixedm_status fixedm_attn_fwd(const fixedm_bounds_t* bounds, fixedm_run_t* run, fixedm_tensor q,
                              const fixedm_tensor* k_chunks, const fixedm_tensor* v_chunks,
                              const int64_t* chunk_len, int32_t n_chunks, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int64_t total = 0;
  fixedm_status st = check_attn_call(bounds, run, q, k_chunks, v_chunks, chunk_len, n_chunks, workspace,
                                     workspace_bytes, &total);
  if (st != FIXEDM_OK) return st;
  if (total == 0) return FIXEDM_OK;
  const AttnArgs a = attn_args(bounds, q, workspace);
  st = enqueue_attn(a, bounds->p, k_chunks, v_chunks, chunk_len, n_chunks, run->kv_visited, nullptr,
                    static_cast<hipStream_t>(stream));
  if (st != FIXEDM_OK) return st;
  run->kv_visited += total;
  run->calls += 1;
  return FIXEDM_OK;
}

fixedm_status fixedm_attn_fwd_final(const fixedm_bounds_t* bounds, fixedm_run_t* run, fixedm_tensor q,
                                    const fixedm_tensor* k_chunks, const fixedm_tensor* v_chunks,
                                    const int64_t* chunk_len, int32_t n_chunks, void* workspace,
                                    size_t workspace_bytes, fixedm_tensor out, int32_t out_dtype, float* lse,
                                    void* stream) {
  int64_t total = 0;
  fixedm_status st = check_attn_call(bounds, run, q, k_chunks, v_chunks, chunk_len, n_chunks, workspace,
                                     workspace_bytes, &total, true);
  if (st != FIXEDM_OK) return st;
  const fixedm_problem& p = bounds->p;
  if ((st = check_out_call(p, out, out_dtype, lse)) != FIXEDM_OK) return st;
  if (run->kv_visited + total != p.sk_total) return FIXEDM_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FinalizeArgs f = finalize_args(p, workspace, out, out_dtype, lse);
  if (total == 0 || p.dtype != FIXEDM_BF16) {
    // nothing left to fold, or the fp32 path: fold, then the finalize kernel
    if (total > 0) {
      const AttnArgs a = attn_args(bounds, q, workspace);
      st = enqueue_attn(a, p, k_chunks, v_chunks, chunk_len, n_chunks, run->kv_visited, nullptr, s);
      if (st != FIXEDM_OK) return st;
    }
    if (launch_finalize(f, s) != hipSuccess) return FIXEDM_ERR_HIP;
  } else {
    AttnArgs a = attn_args(bounds, q, workspace);
    AttnArgs fin;
    memset(&fin, 0, sizeof fin);
    fin.out_dtype = out_dtype;
    fin.out = const_cast<void*>(out.ptr);
    fin.o_sb = out.stride_b; fin.o_ss = out.stride_s; fin.o_sh = out.stride_h;
    fin.lse = lse;
    st = enqueue_attn(a, p, k_chunks, v_chunks, chunk_len, n_chunks, run->kv_visited, &fin, s);
    if (st != FIXEDM_OK) return st;
    if (a.parts > 1) {
      // the split tail tiles left their parts in the workspace: merge and write those tiles
      FinalizeArgs ft = f;
      ft.tile_begin = a.n_whole;
      if (launch_finalize(ft, s) != hipSuccess) return FIXEDM_ERR_HIP;
    }
  }
  run->kv_visited += total;
  run->calls += 1;
  run->finalized = 1;
  return FIXEDM_OK;
}

fixedm_status fixedm_finalize(const fixedm_bounds_t* bounds, const fixedm_run_t* run, const void* workspace,
                              size_t workspace_bytes, fixedm_tensor out, int32_t out_dtype, float* lse,
                              void* stream) {
  fixedm_status st = check_descriptor(bounds);
  if (st != FIXEDM_OK) return st;
  if (run == nullptr || workspace == nullptr) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fixedm_workspace_bytes(&bounds->p)) return FIXEDM_ERR_INVALID_ARGUMENT;
  if (run->token != bounds->token) return FIXEDM_ERR_BOUNDS_MISMATCH;
  if (((uintptr_t)workspace & 255) != 0) return FIXEDM_ERR_INVALID_ARGUMENT;
  const fixedm_problem& p = bounds->p;
  if ((st = check_out_call(p, out, out_dtype, lse)) != FIXEDM_OK) return st;
  if (run->kv_visited != p.sk_total || run->finalized != 0) return FIXEDM_ERR_STATE;
  const FinalizeArgs a = finalize_args(p, workspace, out, out_dtype, lse);
  if (launch_finalize(a, static_cast<hipStream_t>(stream)) != hipSuccess) return FIXEDM_ERR_HIP;
  return FIXEDM_OK;
}

}  // extern "C"
