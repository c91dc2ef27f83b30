// Host side of the C ABI declared in include/fa.h: argument validation, dispatch,
// status strings and the thread-local last-error message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

thread_local std::string g_err;

fa_status fail(fa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

fa_status ok() {
  g_err.clear();
  return FA_OK;
}

constexpr int64_t kMaxPos = 0x7fffffffLL;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The forward, backward and decode kernels tile 64- and 128-blocks; the table writers
// classify any power-of-two block from 1 to 128 (the builder's wavefront walk covers
// up to 128 rows and columns of a block).
bool block_ok(int32_t b) { return b == 64 || b == 128; }
bool table_block_ok(int32_t b) { return b >= 1 && b <= 128 && (b & (b - 1)) == 0; }

// Largest relative-position radius: 2R + 1 table entries per head stay below 2^31.
constexpr int32_t kMaxRelposRadius = (1 << 30) - 1;

// Largest block grid B * H * NQB * NKB: list positions and pointers are int32.
constexpr int64_t kMaxGridBlocks = 0x7fffffffLL;

// Rewrites a valid postfix program so that every and/or node evaluates first the
// operand whose evaluation needs the deeper stack (and/or commute, leaves have no side
// effects, so the mask is the same).  A tree of L leaves then needs a stack of at most
// floor(log2 L) + 1 values: 4 for the 8 leaves of a 16-node program.  Returns that
// depth.
int reorder_program(const fa_mask_desc& m, int32_t* op, int32_t* arg) {
  struct Node { int op, arg, left, right, need; };
  Node nodes[FA_MASK_MAX_NODES];
  int st[FA_MASK_MAX_NODES], sp = 0;
  for (int t = 0; t < m.n; ++t) {
    Node& x = nodes[t];
    x.op = m.node[t].op;
    x.arg = m.node[t].arg;
    x.left = x.right = -1;
    x.need = 1;
    if (x.op == FA_M_AND || x.op == FA_M_OR) {
      x.right = st[--sp];
      x.left = st[--sp];
      const int a = nodes[x.left].need, b = nodes[x.right].need;
      x.need = a == b ? a + 1 : std::max(a, b);
    }
    st[sp++] = t;
  }
  int n = 0;
  auto emit = [&](auto&& self, int t) -> void {
    const Node& x = nodes[t];
    if (x.left >= 0) {
      const bool swap = nodes[x.right].need > nodes[x.left].need;
      self(self, swap ? x.right : x.left);
      self(self, swap ? x.left : x.right);
    }
    op[n] = x.op;
    arg[n] = x.arg;
    ++n;
  };
  emit(emit, st[0]);
  return nodes[st[0]].need;
}

// Validates the postfix program; fills the kernel-side copy.
fa_status check_program(const fa_mask_desc& m, fa::MaskProg* out) {
  if (m.n < 1 || m.n > FA_MASK_MAX_NODES)
    return fail(FA_ERR_MASK_SPEC, "mask program must have 1..%d nodes (got %d)", FA_MASK_MAX_NODES, m.n);
  int depth = 0;
  int has_doc = 0;
  for (int t = 0; t < m.n; ++t) {
    const int op = m.node[t].op;
    const int a = m.node[t].arg;
    switch (op) {
      case FA_M_CAUSAL:
        depth++;
        break;
      case FA_M_SWA:
        if (a < 1) return fail(FA_ERR_MASK_SPEC, "node %d: sliding window W must be >= 1 (got %d)", t, a);
        depth++;
        break;
      case FA_M_DOC:
        has_doc = 1;
        depth++;
        break;
      case FA_M_PREFIX:
        if (a < 0) return fail(FA_ERR_MASK_SPEC, "node %d: prefix length P must be >= 0 (got %d)", t, a);
        depth++;
        break;
      case FA_M_AND:
      case FA_M_OR:
        if (depth < 2) return fail(FA_ERR_MASK_SPEC, "node %d: and/or needs two operands", t);
        depth--;
        break;
      default:
        return fail(FA_ERR_MASK_SPEC, "node %d: unknown mask op %d", t, op);
    }
  }
  if (depth != 1) return fail(FA_ERR_MASK_SPEC, "mask program leaves %d values on the stack (expected 1)", depth);
  if (out) {
    out->n = m.n;
    for (int t = 0; t < FA_MASK_MAX_NODES; ++t) out->op[t] = out->arg[t] = 0;
    if (reorder_program(m, out->op, out->arg) > fa::kMaskStackMax)
      return fail(FA_ERR_MASK_SPEC, "mask program needs a deeper stack than %d", fa::kMaskStackMax);
    out->has_doc = has_doc;
    // An and-only tree of interval leaves is one key interval per row: causal and window
    // bound it above by i, the window below by i - W + 1, prefixes above by max(P-1, i).
    bool and_only = true;
    int wmin = 0, hi_self = 0, pmin = -1;
    for (int t = 0; t < m.n; ++t) {
      const int op = m.node[t].op, a = m.node[t].arg;
      if (op == FA_M_OR) and_only = false;
      if (op == FA_M_CAUSAL) hi_self = 1;
      if (op == FA_M_SWA) {
        hi_self = 1;
        wmin = wmin == 0 ? a : std::min(wmin, a);
      }
      if (op == FA_M_PREFIX) pmin = pmin < 0 ? a : std::min(pmin, a);
    }
    out->mk = and_only ? (has_doc ? fa::MK_INTERVAL_DOC : fa::MK_INTERVAL) : fa::MK_GENERIC;
    out->wmin = wmin;
    out->hi_self = hi_self;
    out->pmin = pmin;
  }
  return FA_OK;
}

// Geometry and mask checks shared by the builder and the forward.
fa_status check_mask_geometry(const fa_block_mask* bm, fa::MaskProg* prog) {
  if (!table_block_ok(bm->block_q) || !table_block_ok(bm->block_kv))
    return fail(FA_ERR_UNSUPPORTED, "block sizes must be powers of two from 1 to 128 (got %d x %d)", bm->block_q,
                bm->block_kv);
  if (bm->B < 1 || bm->H < 1) return fail(FA_ERR_SHAPE, "table extents B, H must be >= 1 (got %d, %d)", bm->B, bm->H);
  if (bm->q_len < 0 || bm->kv_len < 0 || bm->q_offset < 0)
    return fail(FA_ERR_SHAPE, "q_len, kv_len and q_offset must be >= 0");
  if (bm->q_offset + bm->q_len > kMaxPos || bm->kv_len > kMaxPos)
    return fail(FA_ERR_SHAPE, "positions must stay below 2^31");
  const int64_t nqb = cdiv(bm->q_len, bm->block_q), nkb = cdiv(bm->kv_len, bm->block_kv);
  if (nqb > 0 && nkb > 0 && (int64_t)bm->B * bm->H > kMaxGridBlocks / nqb / nkb)
    return fail(FA_ERR_SHAPE, "B*H*NQB*NKB = %d*%d*%lld*%lld blocks exceed the 32-bit list positions", bm->B, bm->H,
                (long long)nqb, (long long)nkb);
  fa_status s = check_program(bm->mask, prog);
  if (s != FA_OK) return s;
  if (prog->has_doc) {
    const fa_mask_desc& m = bm->mask;
    if (!m.doc_ids) return fail(FA_ERR_NULL, "document rule needs doc_ids");
    if (m.doc_batch != 1 && m.doc_batch != bm->B)
      return fail(FA_ERR_MASK_SPEC, "doc_batch (%d) must be 1 or equal to the table batch extent B (%d)", m.doc_batch,
                  bm->B);
    if (m.doc_len < bm->q_offset + bm->q_len || m.doc_len < bm->kv_len)
      return fail(FA_ERR_SHAPE, "doc_len (%lld) must cover q_offset + q_len and kv_len", (long long)m.doc_len);
  }
  return FA_OK;
}

fa::DocRef doc_ref(const fa_block_mask* bm, const fa::MaskProg& prog) {
  fa::DocRef d;
  d.ids = prog.has_doc ? bm->mask.doc_ids : nullptr;
  d.batch = bm->mask.doc_batch < 1 ? 1 : bm->mask.doc_batch;
  d.len = bm->mask.doc_len;
  return d;
}

int num_cus_of_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

struct FwdPlan {
  fa::FwdParams p;
  bool decode;
  bool per_head;   // decode path in its per-head view (fa::decode_per_head)
  size_t ws;
};

fa_status plan_forward(const fa_fwd_args* a, FwdPlan* plan) {
  if (!a) return fail(FA_ERR_NULL, "args is NULL");
  if (!a->q || !a->k || !a->v || !a->o || !a->lse) return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  // rows move in 16-byte chunks (global_load_lds_dwordx4 and 16-byte loads and stores)
  if (((uintptr_t)a->q | (uintptr_t)a->k | (uintptr_t)a->v | (uintptr_t)a->o) & 15)
    return fail(FA_ERR_SHAPE, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)a->lse & 3) return fail(FA_ERR_SHAPE, "lse must be 4-byte aligned");
  if (!a->bm) return fail(FA_ERR_NULL, "bm (block tables) is NULL");
  const fa_block_mask* bm = a->bm;
  if (a->d != 64 && a->d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %d)", a->d);
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1) return fail(FA_ERR_SHAPE, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv != 0) return fail(FA_ERR_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", a->Hq, a->Hkv);
  if (a->q_len < 0 || a->kv_len < 0) return fail(FA_ERR_SHAPE, "q_len and kv_len must be >= 0");
  fa::MaskProg prog;
  fa_status s = check_mask_geometry(bm, &prog);
  if (s != FA_OK) return s;
  if (!block_ok(bm->block_q) || !block_ok(bm->block_kv))
    return fail(FA_ERR_UNSUPPORTED, "the attention kernels run on 64- or 128-blocks (tables of %d x %d)", bm->block_q,
                bm->block_kv);
  if (bm->q_len != a->q_len || bm->kv_len != a->kv_len)
    return fail(FA_ERR_MASK_MISMATCH, "block tables were built for q_len=%lld kv_len=%lld, forward has %lld, %lld",
                (long long)bm->q_len, (long long)bm->kv_len, (long long)a->q_len, (long long)a->kv_len);
  if (bm->B != 1 && bm->B != a->B)
    return fail(FA_ERR_MASK_MISMATCH, "table batch extent %d is neither 1 nor B=%d", bm->B, a->B);
  if (bm->H != 1 && bm->H != a->Hq)
    return fail(FA_ERR_MASK_MISMATCH, "table head extent %d is neither 1 nor Hq=%d", bm->H, a->Hq);
  if (prog.has_doc && bm->mask.doc_batch != 1 && bm->mask.doc_batch != a->B)
    return fail(FA_ERR_MASK_MISMATCH, "doc_batch %d does not match B=%d", bm->mask.doc_batch, a->B);
  if (!bm->kv_num || !bm->kv_ptr || !bm->kv_idx || !bm->full_kv_num || !bm->full_kv_ptr || !bm->full_kv_idx)
    return fail(FA_ERR_NULL, "kv-side block tables must be non-NULL");
  const fa_score_desc& sd = a->score;
  switch (sd.kind) {
    case FA_S_IDENTITY:
      break;
    case FA_S_ALIBI:
      if (!sd.alibi_slopes) return fail(FA_ERR_NULL, "ALiBi needs alibi_slopes");
      break;
    case FA_S_SOFTCAP:
      if (!(sd.softcap > 0.f) || !std::isfinite(sd.softcap))
        return fail(FA_ERR_UNSUPPORTED, "softcap must be a finite value > 0");
      break;
    case FA_S_RELPOS:
      if (!sd.relpos) return fail(FA_ERR_NULL, "relative-position bias needs its table");
      if (sd.relpos_radius < 0 || sd.relpos_radius > kMaxRelposRadius)
        return fail(FA_ERR_UNSUPPORTED, "relpos_radius must be in [0, %d] (got %d)", kMaxRelposRadius,
                    sd.relpos_radius);
      break;
    default:
      return fail(FA_ERR_UNSUPPORTED, "unknown score_mod kind %d", sd.kind);
  }
  float scale = a->scale;
  if (std::isnan(scale) || std::isinf(scale)) return fail(FA_ERR_SHAPE, "scale must be finite");
  if (scale <= 0.f) scale = 1.0f / std::sqrt((float)a->d);

  fa::FwdParams& p = plan->p;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = static_cast<uint16_t*>(a->o);
  p.lse = a->lse;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.g = a->Hq / a->Hkv;
  p.d = a->d;
  p.q_len = a->q_len;
  p.kv_len = a->kv_len;
  p.q_offset = bm->q_offset;
  p.scale = scale;
  p.score.kind = sd.kind;
  p.score.softcap = sd.softcap;
  p.score.slopes = sd.alibi_slopes;
  p.score.table = sd.relpos;
  p.score.radius = sd.relpos_radius;
  p.prog = prog;
  p.doc = doc_ref(bm, prog);
  p.tab.num = bm->kv_num;
  p.tab.ptr = bm->kv_ptr;
  p.tab.idx = bm->kv_idx;
  p.tab.fnum = bm->full_kv_num;
  p.tab.fptr = bm->full_kv_ptr;
  p.tab.fidx = bm->full_kv_idx;
  p.tab.qnum = bm->q_num;
  p.tab.qptr = bm->q_ptr;
  p.tab.qidx = bm->q_idx;
  p.tab.qfnum = bm->full_q_num;
  p.tab.qfptr = bm->full_q_ptr;
  p.tab.qfidx = bm->full_q_idx;
  p.tab.order = bm->order;
  p.tab.tB = bm->B;
  p.tab.tH = bm->H;
  p.tab.nqb = (int32_t)cdiv(a->q_len, bm->block_q);
  p.tab.nkb = (int32_t)cdiv(a->kv_len, bm->block_kv);
  if (bm->order && p.tab.nqb > fa::kOrderMaxRows)
    return fail(FA_ERR_UNSUPPORTED, "a work order needs at most %d query blocks", fa::kOrderMaxRows);
  p.tab.bq = bm->block_q;
  p.tab.bk = bm->block_kv;
  p.nsplit = 1;
  p.ws = nullptr;
  p.pt = nullptr;
  p.pt_stride = 0;
  p.page_shift = 0;
  p.num_pages = 0;
  p.kv_group = 1;
  fa::FwdParams v = p;
  plan->per_head = a->q_len > 0 && !fa::decode_eligible(p) && fa::decode_per_head(v);
  plan->decode = a->q_len > 0 && (fa::decode_eligible(p) || plan->per_head);
  plan->ws = 0;
  if (plan->decode) {
    const fa::FwdParams& d = plan->per_head ? v : p;
    p.nsplit = fa::decode_splits(d, num_cus_of_current_device());
    plan->ws = fa::decode_workspace_bytes(d, p.nsplit);
  }
  return FA_OK;
}

fa_status launch_planned(const FwdPlan& plan, const fa_fwd_args* args, fa_stream_t stream) {
  if (args->q_len == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  fa::FwdParams lp = plan.p;
  if (plan.per_head) fa::decode_per_head(lp);
  hipError_t e = plan.decode ? fa::launch_decode(lp, st) : fa::launch_prefill(lp, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------------
// Scratch of fa_forward_noalloc: the split-KV partial states live in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` only names the symbol: its
// device address on the current GPU comes from hipGetSymbolAddress, looked up once per
// device (with that device current) on the first call there, and only that address is
// ever handed to kernels.
// ---------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "device %d is beyond the %d devices with a scratch slot", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: inconsistent or unsupported sizes";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim, block size or score kind outside the menu";
    case FA_ERR_MASK_SPEC: return "FA_ERR_MASK_SPEC: malformed mask program or parameter";
    case FA_ERR_MASK_MISMATCH: return "FA_ERR_MASK_MISMATCH: block tables do not match the forward's shapes";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
  }
  return "unknown fa_status";
}

const char* fa_last_error_message(void) { return g_err.c_str(); }

fa_status fa_block_mask_sizes(const fa_block_mask* bm, int64_t* rows, int64_t* cols, int64_t* idx_capacity,
                              size_t* workspace_bytes) {
  if (!bm) return fail(FA_ERR_NULL, "bm is NULL");
  if (!table_block_ok(bm->block_q) || !table_block_ok(bm->block_kv))
    return fail(FA_ERR_UNSUPPORTED, "block sizes must be powers of two from 1 to 128 (got %d x %d)", bm->block_q,
                bm->block_kv);
  if (bm->B < 1 || bm->H < 1) return fail(FA_ERR_SHAPE, "table extents B, H must be >= 1");
  if (bm->q_len < 0 || bm->kv_len < 0 || bm->q_offset < 0) return fail(FA_ERR_SHAPE, "negative length or offset");
  if (bm->q_offset + bm->q_len > kMaxPos || bm->kv_len > kMaxPos) return fail(FA_ERR_SHAPE, "positions must stay below 2^31");
  const int64_t nqb = cdiv(bm->q_len, bm->block_q);
  const int64_t nkb = cdiv(bm->kv_len, bm->block_kv);
  if (rows) *rows = (int64_t)bm->B * bm->H * nqb;
  if (cols) *cols = (int64_t)bm->B * bm->H * nkb;
  if (idx_capacity) *idx_capacity = (int64_t)bm->B * bm->H * nqb * nkb;
  if (workspace_bytes)
    *workspace_bytes = std::max(fa::build_workspace_bytes(bm->B, nqb, nkb),
                                fa::slice_workspace_bytes((int64_t)bm->B * bm->H, nqb, nkb));
  return ok();
}

fa_status fa_create_block_mask(fa_block_mask* bm, void* workspace, size_t ws_bytes, fa_stream_t stream) {
  if (!bm) return fail(FA_ERR_NULL, "bm is NULL");
  fa::MaskProg prog;
  fa_status s = check_mask_geometry(bm, &prog);
  if (s != FA_OK) return s;
  if (!bm->kv_num || !bm->kv_ptr || !bm->kv_idx || !bm->full_kv_num || !bm->full_kv_ptr || !bm->full_kv_idx)
    return fail(FA_ERR_NULL, "the six kv-side table pointers must be non-NULL");
  const int nq_set = (bm->q_num != nullptr) + (bm->q_ptr != nullptr) + (bm->q_idx != nullptr) +
                     (bm->full_q_num != nullptr) + (bm->full_q_ptr != nullptr) + (bm->full_q_idx != nullptr);
  if (nq_set != 0 && nq_set != 6)
    return fail(FA_ERR_NULL, "the six q-side table pointers must be all set or all NULL");
  const int64_t nqb = cdiv(bm->q_len, bm->block_q);
  const int64_t nkb = cdiv(bm->kv_len, bm->block_kv);
  const size_t need = fa::build_workspace_bytes(bm->B, nqb, nkb);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(FA_ERR_WORKSPACE, "builder workspace needs %zu bytes (got %zu)", need, workspace ? ws_bytes : (size_t)0);
  if (nqb > 0x7fffffff || nkb > 0x7fffffff) return fail(FA_ERR_SHAPE, "too many blocks");
  if (bm->order && nqb > fa::kOrderMaxRows)
    return fail(FA_ERR_UNSUPPORTED, "a work order needs at most %d query blocks", fa::kOrderMaxRows);
  fa::BuildParams p;
  p.prog = prog;
  p.doc = doc_ref(bm, prog);
  p.tB = bm->B;
  p.tH = bm->H;
  p.q_len = bm->q_len;
  p.kv_len = bm->kv_len;
  p.q_offset = bm->q_offset;
  p.bq = bm->block_q;
  p.bk = bm->block_kv;
  p.nqb = (int32_t)nqb;
  p.nkb = (int32_t)nkb;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.grid = ws;
  const size_t grid_bytes = (size_t)(bm->B * nqb * nkb + 255) & ~(size_t)255;
  p.qstat = reinterpret_cast<int32_t*>(ws + grid_bytes);
  p.kstat = p.qstat + (size_t)bm->B * nqb * 2;
  p.kv_num = bm->kv_num;
  p.kv_ptr = bm->kv_ptr;
  p.kv_idx = bm->kv_idx;
  p.full_kv_num = bm->full_kv_num;
  p.full_kv_ptr = bm->full_kv_ptr;
  p.full_kv_idx = bm->full_kv_idx;
  p.q_num = bm->q_num;
  p.q_ptr = bm->q_ptr;
  p.q_idx = bm->q_idx;
  p.full_q_num = bm->full_q_num;
  p.full_q_ptr = bm->full_q_ptr;
  p.full_q_idx = bm->full_q_idx;
  p.order = bm->order;
  hipError_t e = fa::launch_build(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "block-mask build launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_forward_workspace_size(const fa_fwd_args* args, size_t* bytes) {
  FwdPlan plan;
  fa_status s = plan_forward(args, &plan);
  if (s != FA_OK) return s;
  if (!bytes) return fail(FA_ERR_NULL, "bytes is NULL");
  *bytes = plan.ws;
  return ok();
}

fa_status fa_forward(const fa_fwd_args* args, fa_stream_t stream) {
  return fa_forward_paged(args, nullptr, stream);
}

namespace {

// ws: the minimum workspace (row sums dO . O); ds_ws: the stored-gradient part that may
// follow it (0 when this shape always recomputes the gradients in the dQ pass)
fa_status plan_backward(const fa_bwd_args* a, fa::BwdParams* bp, size_t* ws, size_t* ds_ws) {
  if (!a) return fail(FA_ERR_NULL, "args is NULL");
  FwdPlan plan;
  fa_status s = plan_forward(a->fwd, &plan);
  if (s != FA_OK) return s;
  const fa_block_mask* bm = a->fwd->bm;
  if (!bm->q_num || !bm->q_ptr || !bm->q_idx || !bm->full_q_num || !bm->full_q_ptr || !bm->full_q_idx)
    return fail(FA_ERR_NULL, "the backward needs the q-side block tables");
  if (!a->dout || !a->dq || !a->dk || !a->dv) return fail(FA_ERR_NULL, "dout, dq, dk and dv must be non-NULL");
  if (((uintptr_t)a->dout | (uintptr_t)a->dq | (uintptr_t)a->dk | (uintptr_t)a->dv) & 15)
    return fail(FA_ERR_SHAPE, "dout, dq, dk and dv must be 16-byte aligned");
  bp->f = plan.p;
  bp->dout = static_cast<const uint16_t*>(a->dout);
  bp->dq = a->dq;
  bp->dk = a->dk;
  bp->dv = a->dv;
  bp->ndelta = nullptr;
  bp->lrow = nullptr;
  bp->ds = nullptr;
  const int kind = a->fwd->score.kind;
  if (a->dslopes && kind != FA_S_ALIBI)
    return fail(FA_ERR_UNSUPPORTED, "dslopes is the gradient of ALiBi slopes; the score kind is %d", kind);
  if (a->dtable && kind != FA_S_RELPOS)
    return fail(FA_ERR_UNSUPPORTED, "dtable is the gradient of a relative-position table; the score kind is %d", kind);
  if (a->dtable && a->fwd->score.relpos_radius > fa::kRelGradMaxRadius)
    return fail(FA_ERR_UNSUPPORTED, "the position-table gradient supports radius <= %d (got %d)",
                fa::kRelGradMaxRadius, a->fwd->score.relpos_radius);
  bp->dslopes = a->dslopes;
  bp->dtable = a->dtable;
  *ws = fa::backward_workspace_min_bytes(plan.p);
  *ds_ws = fa::backward_ds_bytes(plan.p, a->dslopes != nullptr || a->dtable != nullptr);
  return FA_OK;
}

}  // namespace

fa_status fa_backward_workspace_size(const fa_bwd_args* args, size_t* bytes) {
  fa::BwdParams bp;
  size_t ws = 0, ds_ws = 0;
  fa_status s = plan_backward(args, &bp, &ws, &ds_ws);
  if (s != FA_OK) return s;
  if (!bytes) return fail(FA_ERR_NULL, "bytes is NULL");
  *bytes = ws + ds_ws;
  return ok();
}

fa_status fa_backward_workspace_min_size(const fa_bwd_args* args, size_t* bytes) {
  fa::BwdParams bp;
  size_t ws = 0, ds_ws = 0;
  fa_status s = plan_backward(args, &bp, &ws, &ds_ws);
  if (s != FA_OK) return s;
  if (!bytes) return fail(FA_ERR_NULL, "bytes is NULL");
  *bytes = ws;
  return ok();
}

fa_status fa_backward(const fa_bwd_args* args, fa_stream_t stream) {
  fa::BwdParams bp;
  size_t ws = 0, ds_ws = 0;
  fa_status s = plan_backward(args, &bp, &ws, &ds_ws);
  if (s != FA_OK) return s;
  if (ws > 0) {
    if (!args->workspace || args->ws_bytes < ws)
      return fail(FA_ERR_WORKSPACE, "backward workspace needs %zu bytes (got %zu)", ws,
                  args->workspace ? args->ws_bytes : (size_t)0);
    if (((uintptr_t)args->workspace & 255) != 0)
      return fail(FA_ERR_WORKSPACE, "backward workspace must be 256-byte aligned");
    bp.ndelta = static_cast<float*>(args->workspace);
    bp.lrow = bp.ndelta + ws / (2 * sizeof(float));   // the second 256-byte-aligned half
    if (ds_ws > 0 && args->ws_bytes >= ws + ds_ws)   // ws is a multiple of 256 bytes
      bp.ds = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(args->workspace) + ws);
  }
  hipError_t e = fa::launch_backward(bp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_forward_paged(const fa_fwd_args* args, const fa_paged_kv* kv, fa_stream_t stream) {
  FwdPlan plan;
  fa_status s = plan_forward(args, &plan);
  if (s != FA_OK) return s;
  if (kv) {
    if (!kv->page_table) return fail(FA_ERR_NULL, "page_table is NULL");
    const int32_t ps = kv->page_size;
    if (ps < 16 || ps > 65536 || (ps & (ps - 1)) != 0)
      return fail(FA_ERR_UNSUPPORTED, "page_size must be a power of two in [16, 65536] (got %d)", ps);
    const int64_t pages = (args->kv_len + ps - 1) / ps;
    if (kv->pt_stride < pages)
      return fail(FA_ERR_SHAPE, "pt_stride %lld is below the %lld pages of kv_len", (long long)kv->pt_stride,
                  (long long)pages);
    if (kv->num_pages < 1 || kv->num_pages > 0x7fffffffLL)
      return fail(FA_ERR_SHAPE, "num_pages must be in [1, 2^31 - 1]");
    if (args->q_len > 0 && !plan.decode)
      return fail(FA_ERR_UNSUPPORTED, "a paged KV cache is read by the short-query path only: "
                  "(Hq/Hkv) * q_len <= 16 (q_len <= 16 with per-head tables), one query block and "
                  "block_kv == 128");
    plan.p.pt = kv->page_table;
    plan.p.pt_stride = kv->pt_stride;
    plan.p.page_shift = __builtin_ctz((unsigned)ps);
    plan.p.num_pages = kv->num_pages;
  }
  if (plan.ws > 0) {
    if (!args->workspace || args->ws_bytes < plan.ws)
      return fail(FA_ERR_WORKSPACE, "forward workspace needs %zu bytes (got %zu)", plan.ws,
                  args->workspace ? args->ws_bytes : (size_t)0);
    if ((uintptr_t)args->workspace & 15) return fail(FA_ERR_WORKSPACE, "forward workspace must be 16-byte aligned");
    plan.p.ws = static_cast<float*>(args->workspace);
  }
  return launch_planned(plan, args, stream);
}

fa_status fa_forward_noalloc(const fa_fwd_args* args, fa_stream_t stream) {
  FwdPlan plan;
  fa_status s = plan_forward(args, &plan);
  if (s != FA_OK) return s;
  if (plan.ws > (size_t)FA_NOALLOC_SCRATCH_BYTES)
    return fail(FA_ERR_WORKSPACE, "this forward needs %zu bytes of split-KV scratch; the static scratch holds %zu",
                plan.ws, (size_t)FA_NOALLOC_SCRATCH_BYTES);
  if (plan.ws > 0 && args->q_len > 0) {
    void* ptr = nullptr;
    s = scratch_of_current_device(&ptr);
    if (s != FA_OK) return s;
    plan.p.ws = static_cast<float*>(ptr);
  }
  return launch_planned(plan, args, stream);
}

fa_status fa_block_mask_from_indices(fa_block_mask* bm, const int32_t* sel, int32_t k, void* workspace,
                                     size_t ws_bytes, fa_stream_t stream) {
  if (!bm) return fail(FA_ERR_NULL, "bm is NULL");
  fa::MaskProg prog;
  fa_status s = check_mask_geometry(bm, &prog);
  if (s != FA_OK) return s;
  if (!bm->kv_num || !bm->kv_ptr || !bm->kv_idx || !bm->full_kv_num || !bm->full_kv_ptr || !bm->full_kv_idx)
    return fail(FA_ERR_NULL, "kv-side table pointers must be non-NULL");
  const int nq_set = (bm->q_num != nullptr) + (bm->q_ptr != nullptr) + (bm->q_idx != nullptr) +
                     (bm->full_q_num != nullptr) + (bm->full_q_ptr != nullptr) + (bm->full_q_idx != nullptr);
  if (nq_set != 0 && nq_set != 6) return fail(FA_ERR_NULL, "q-side tables must be all set or all NULL");
  const bool qside = nq_set == 6;
  const int64_t nqb = cdiv(bm->q_len, bm->block_q), nkb = cdiv(bm->kv_len, bm->block_kv);
  const int64_t tBH = (int64_t)bm->B * bm->H;
  if (k < 0) return fail(FA_ERR_SHAPE, "candidate count k must be >= 0 (got %d)", k);
  if (k > 0 && tBH * nqb > 0 && !sel) return fail(FA_ERR_NULL, "sel is NULL");
  if (tBH * nqb * nkb > 0x7fffffffLL || tBH * (nqb + nkb) > 0x7fffffffLL || tBH * nqb * (int64_t)k > (1LL << 40))
    return fail(FA_ERR_SHAPE, "tables too large for 32-bit indices");
  if (bm->order && nqb > fa::kOrderMaxRows)
    return fail(FA_ERR_UNSUPPORTED, "a work order needs at most %d query blocks", fa::kOrderMaxRows);
  const size_t need = fa::slice_workspace_bytes(tBH, nqb, nkb);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(FA_ERR_WORKSPACE, "selector tables need %zu bytes of workspace (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  if (((uintptr_t)workspace & 15) != 0) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  fa::SelectParams sp;
  fa::BuildParams& p = sp.d;
  p.prog = prog;
  p.doc = doc_ref(bm, prog);
  p.tB = (int32_t)tBH;
  p.tH = 1;
  p.q_len = bm->q_len;
  p.kv_len = bm->kv_len;
  p.q_offset = bm->q_offset;
  p.bq = bm->block_q;
  p.bk = bm->block_kv;
  p.nqb = (int32_t)nqb;
  p.nkb = (int32_t)nkb;
  p.grid = static_cast<uint8_t*>(workspace);
  p.qstat = p.kstat = nullptr;
  p.kv_num = bm->kv_num;
  p.kv_ptr = bm->kv_ptr;
  p.kv_idx = bm->kv_idx;
  p.full_kv_num = bm->full_kv_num;
  p.full_kv_ptr = bm->full_kv_ptr;
  p.full_kv_idx = bm->full_kv_idx;
  p.q_num = qside ? bm->q_num : nullptr;
  p.q_ptr = qside ? bm->q_ptr : nullptr;
  p.q_idx = qside ? bm->q_idx : nullptr;
  p.full_q_num = qside ? bm->full_q_num : nullptr;
  p.full_q_ptr = qside ? bm->full_q_ptr : nullptr;
  p.full_q_idx = qside ? bm->full_q_idx : nullptr;
  p.order = bm->order;
  sp.sel = sel;
  sp.k = k;
  sp.H = bm->H;
  hipError_t e = fa::launch_select(sp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "selector table launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_block_mask_slice(const fa_block_mask* src, fa_block_mask* dst, void* workspace, size_t ws_bytes,
                              fa_stream_t stream) {
  if (!src || !dst) return fail(FA_ERR_NULL, "src and dst must be non-NULL");
  fa::MaskProg prog;
  fa_status s = check_mask_geometry(src, &prog);
  if (s != FA_OK) return s;
  fa::MaskProg prog_dst;
  s = check_mask_geometry(dst, &prog_dst);
  if (s != FA_OK) return s;
  const fa_mask_desc &ms = src->mask, &md = dst->mask;
  bool same = ms.n == md.n &&
              (!prog.has_doc || (ms.doc_ids == md.doc_ids && ms.doc_batch == md.doc_batch && ms.doc_len == md.doc_len));
  for (int t = 0; same && t < ms.n; ++t)
    same = ms.node[t].op == md.node[t].op &&
           ((ms.node[t].op != FA_M_SWA && ms.node[t].op != FA_M_PREFIX) || ms.node[t].arg == md.node[t].arg);
  if (!same) return fail(FA_ERR_MASK_MISMATCH, "dst must carry the same mask rule (program and document IDs) as src");
  if (src->B != dst->B || src->H != dst->H || src->block_q != dst->block_q || src->block_kv != dst->block_kv)
    return fail(FA_ERR_MASK_MISMATCH, "dst must have the table extents and block sizes of src");
  if (dst->kv_len > src->kv_len || dst->q_offset < src->q_offset ||
      dst->q_offset + dst->q_len > src->q_offset + src->q_len)
    return fail(FA_ERR_SHAPE,
                "slice rows [%lld, %lld) x keys [0, %lld) leave the prebuilt rows [%lld, %lld) x keys [0, %lld); "
                "a longer context needs tables built for it",
                (long long)dst->q_offset, (long long)(dst->q_offset + dst->q_len), (long long)dst->kv_len,
                (long long)src->q_offset, (long long)(src->q_offset + src->q_len), (long long)src->kv_len);
  const int64_t delta = dst->q_offset - src->q_offset;
  const int64_t nqb = cdiv(dst->q_len, dst->block_q), nkb = cdiv(dst->kv_len, dst->block_kv);
  const int64_t nqb_src = cdiv(src->q_len, src->block_q), nkb_src = cdiv(src->kv_len, src->block_kv);
  const bool aligned = delta % dst->block_q == 0;
  const bool inside_one = nqb == 1 && delta / dst->block_q == (delta + dst->q_len - 1) / dst->block_q;
  if (nqb > 0 && !aligned && !inside_one)
    return fail(FA_ERR_SHAPE,
                "each new query block must be one prebuilt query block or lie inside one: q_offset - src.q_offset "
                "(%lld) must be a multiple of block_q, or the rows must fit in one prebuilt block",
                (long long)delta);
  if ((int64_t)src->B * src->H * nqb_src * nkb_src > 0x7fffffffLL ||
      (int64_t)src->B * src->H * (nqb_src + nkb_src) > 0x7fffffffLL)
    return fail(FA_ERR_SHAPE, "prebuilt tables too large for 32-bit indices");
  if (!src->kv_num || !src->kv_ptr || !src->kv_idx || !src->full_kv_num || !src->full_kv_ptr || !src->full_kv_idx)
    return fail(FA_ERR_NULL, "src kv-side tables must be non-NULL");
  if (!dst->kv_num || !dst->kv_ptr || !dst->kv_idx || !dst->full_kv_num || !dst->full_kv_ptr || !dst->full_kv_idx)
    return fail(FA_ERR_NULL, "dst kv-side tables must be non-NULL");
  const int nq_set = (dst->q_num != nullptr) + (dst->q_ptr != nullptr) + (dst->q_idx != nullptr) +
                     (dst->full_q_num != nullptr) + (dst->full_q_ptr != nullptr) + (dst->full_q_idx != nullptr);
  if (nq_set != 0 && nq_set != 6)
    return fail(FA_ERR_NULL, "dst q-side tables must be all set or all NULL");
  const bool qside = nq_set == 6;
  if (dst->order && nqb > fa::kOrderMaxRows)
    return fail(FA_ERR_UNSUPPORTED, "a work order needs at most %d query blocks", fa::kOrderMaxRows);
  const size_t need = fa::slice_workspace_bytes((int64_t)dst->B * dst->H, nqb, nkb);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(FA_ERR_WORKSPACE, "slice workspace needs %zu bytes (got %zu)", need, workspace ? ws_bytes : (size_t)0);
  if (((uintptr_t)workspace & 15) != 0) return fail(FA_ERR_WORKSPACE, "slice workspace must be 16-byte aligned");
  fa::SliceParams sp;
  fa::BuildParams& p = sp.d;
  p.prog = prog;
  p.doc = doc_ref(dst, prog);
  p.tB = src->B * src->H;
  p.tH = 1;
  p.q_len = dst->q_len;
  p.kv_len = dst->kv_len;
  p.q_offset = dst->q_offset;
  p.bq = dst->block_q;
  p.bk = dst->block_kv;
  p.nqb = (int32_t)nqb;
  p.nkb = (int32_t)nkb;
  p.grid = static_cast<uint8_t*>(workspace);
  p.qstat = p.kstat = nullptr;
  p.kv_num = dst->kv_num;
  p.kv_ptr = dst->kv_ptr;
  p.kv_idx = dst->kv_idx;
  p.full_kv_num = dst->full_kv_num;
  p.full_kv_ptr = dst->full_kv_ptr;
  p.full_kv_idx = dst->full_kv_idx;
  p.q_num = qside ? dst->q_num : nullptr;
  p.q_ptr = qside ? dst->q_ptr : nullptr;
  p.q_idx = qside ? dst->q_idx : nullptr;
  p.full_q_num = qside ? dst->full_q_num : nullptr;
  p.full_q_ptr = qside ? dst->full_q_ptr : nullptr;
  p.full_q_idx = qside ? dst->full_q_idx : nullptr;
  p.order = dst->order;
  sp.s_num[0] = src->kv_num;
  sp.s_ptr[0] = src->kv_ptr;
  sp.s_idx[0] = src->kv_idx;
  sp.s_num[1] = src->full_kv_num;
  sp.s_ptr[1] = src->full_kv_ptr;
  sp.s_idx[1] = src->full_kv_idx;
  sp.nqb_src = (int32_t)nqb_src;
  sp.nkb_src = (int32_t)nkb_src;
  sp.r_base = (int32_t)(delta / dst->block_q);
  sp.H = src->H;
  sp.src_q_offset = src->q_offset;
  sp.src_q_len = src->q_len;
  sp.src_kv_len = src->kv_len;
  hipError_t e = fa::launch_slice(sp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "block-mask slice launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
