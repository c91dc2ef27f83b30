// Internal parameter blocks and launchers shared by the host API and the kernels.
// Nothing here is part of the public ABI (include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// How a kernel evaluates the element mask on partial blocks.
enum MaskKind : int32_t {
  MK_INTERVAL = 0,      // and-tree of causal / window / prefix: one key interval per row
  MK_INTERVAL_DOC = 1,  // the same intersected with document equality
  MK_GENERIC = 2        // anything with an or-node: postfix interpreter per element
};

// Stack depth that any valid program reaches once the host has ordered every and/or
// node's operands deeper-first (8 leaves at most, so floor(log2 8) + 1).
constexpr int kMaskStackMax = 4;

// Mask program as passed to kernels (by value, in kernel arguments), operands of each
// and/or node in deeper-first order.
struct MaskProg {
  int32_t n;
  int32_t op[FA_MASK_MAX_NODES];
  int32_t arg[FA_MASK_MAX_NODES];
  int32_t has_doc;
  // interval form (MK_INTERVAL*): allowed keys of global row i are [lo(i), hi(i)] with
  // lo = max(0, i - wmin + 1) if wmin > 0 else 0, hi = i if hi_self, else
  // max(pmin - 1, i) if pmin >= 0, else unbounded
  int32_t mk;
  int32_t wmin;
  int32_t hi_self;
  int32_t pmin;
};

struct DocRef {
  const int32_t* ids;  // [doc_batch, doc_len] or nullptr
  int32_t batch;
  int64_t len;
};

// ---------------------------------------------------------------- builder
struct BuildParams {
  MaskProg prog;
  DocRef doc;
  int32_t tB, tH;
  int64_t q_len, kv_len, q_offset;
  int32_t bq, bk;
  int32_t nqb, nkb;
  uint8_t* grid;      // [tB][nqb][nkb] classes
  int32_t* qstat;     // [tB][nqb][2] doc min/max over the query block
  int32_t* kstat;     // [tB][nkb][2] doc min/max over the KV block
  int32_t *kv_num, *kv_ptr, *kv_idx, *full_kv_num, *full_kv_ptr, *full_kv_idx;
  int32_t *q_num, *q_ptr, *q_idx, *full_q_num, *full_q_ptr, *full_q_idx;
  int32_t* order;     // longest-row-first work order, or nullptr
};

constexpr int kOrderMaxRows = 4096;   // NQB limit of the work order

size_t build_workspace_bytes(int64_t tB, int64_t nqb, int64_t nkb);
hipError_t launch_build(const BuildParams& p, hipStream_t s);

// Row slice of prebuilt tables.  The destination is described as a build of its own
// (d.tB = table B * H, d.tH = 1: every (b', h') row is sliced on its own; d.q_num ==
// nullptr skips the query side; d.grid is the workspace); its rows are source rows
// r_base .. r_base + nqb - 1 of the same (b', h') with columns c < d.nkb.
struct SliceParams {
  BuildParams d;
  const int32_t* s_num[2];   // source kv-side lists: partial, full
  const int32_t* s_ptr[2];
  const int32_t* s_idx[2];
  int32_t nqb_src, nkb_src, r_base;
  int32_t H;                 // table head extent: (b', h') = bh gives doc batch bh / H
  int64_t src_q_offset, src_q_len, src_kv_len;
};
size_t slice_workspace_bytes(int64_t tBH, int64_t nqb, int64_t nkb);
hipError_t launch_slice(const SliceParams& p, hipStream_t s);

// Tables from selector output: d as for the slice (d.grid = workspace); sel is
// [tB = B*H][nqb][k] KV block indices; H gives the doc batch of a table entry.
struct SelectParams {
  BuildParams d;
  const int32_t* sel;
  int32_t k;
  int32_t H;
};
hipError_t launch_select(const SelectParams& p, hipStream_t s);

// ---------------------------------------------------------------- forward
struct ScoreParams {
  int32_t kind;
  float softcap;
  const float* slopes;
  const float* table;
  int32_t radius;
};

struct TableRef {
  const int32_t *num, *ptr, *idx;             // partial list
  const int32_t *fnum, *fptr, *fidx;          // full list
  const int32_t *qnum, *qptr, *qidx;          // q side (columns): partial list
  const int32_t *qfnum, *qfptr, *qfidx;       // q side: full list
  const int32_t* order;                       // per (b', h'): query blocks longest first, or nullptr
  int32_t tB, tH, nqb, nkb, bq, bk;
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int32_t B, Hq, Hkv, g, d;
  int64_t q_len, kv_len, q_offset;
  float scale;
  ScoreParams score;
  MaskProg prog;
  DocRef doc;
  TableRef tab;
  // split-KV decode
  int32_t nsplit;
  float* ws;  // partial states
  // paged K/V (decode path): k and v are [num_pages, Hkv, page_size, d]; pt == nullptr
  // for contiguous K/V
  const int32_t* pt;
  int64_t pt_stride;
  int32_t page_shift;   // log2(page_size)
  int64_t num_pages;
  // decode path: query heads per memory KV head of a unit head (1 normally; g in the
  // per-head view, where every query head is a unit of its own)
  int32_t kv_group;
};

bool decode_eligible(const FwdParams& p);
// Turns p into the per-head view of the decode path (Hkv := Hq, g := 1, kv_group := g)
// when the tables hold a row per query head under GQA and the view is decode-eligible.
bool decode_per_head(FwdParams& p);
int32_t decode_splits(const FwdParams& p, int num_cus);
size_t decode_workspace_bytes(const FwdParams& p, int32_t nsplit);
hipError_t launch_prefill(const FwdParams& p, hipStream_t s);

// ---------------------------------------------------------------- backward
struct BwdParams {
  FwdParams f;            // the forward's inputs, O and LSE (from the forward)
  const uint16_t* dout;   // bf16 [B, Hq, q_len, d]
  float* dq;              // fp32 [B, Hq, q_len, d]
  float* dk;              // fp32 [B, Hkv, kv_len, d]
  float* dv;              // fp32 [B, Hkv, kv_len, d]
  float* ndelta;          // fp32 [B, Hq, q_len] workspace: -rowsum(dO * O)
  float* lrow;            // fp32 [B, Hq, q_len] workspace: the row term of the weights,
                          // (cap log2 e for soft-cap, else 0) - LSE log2 e
  uint16_t* ds;           // bf16 per-pair gradients of every executed block, stored by the
                          // dK/dV pass for the dQ pass, or nullptr (the dQ pass recomputes
                          // them).  Tile [b][h_q][query block][KV block] of 128 x 128
                          // values in the order of the lanes that form them: 16-byte
                          // chunk ((w * 4 + s) * 64 + l) holds key 16 w + (l & 15) for
                          // query rows 32 s + 4 (l >> 4) + (0..3), then those rows + 16
  float* dslopes;         // fp32 [Hq]: gradient of the ALiBi slopes, or nullptr
  float* dtable;          // fp32 [Hq, 2R+1]: gradient of the position table, or nullptr
};
constexpr int kRelGradMaxRadius = 1024;   // position-table gradients: bins kept in LDS
constexpr size_t kDsMaxBytes = (size_t)8 << 30;   // stored gradients: largest workspace part
size_t backward_workspace_min_bytes(const FwdParams& p);
// bytes of the stored-gradient part of the backward workspace (0: not used for this shape)
size_t backward_ds_bytes(const FwdParams& p, bool param_grads);
hipError_t launch_backward(const BwdParams& p, hipStream_t s);
hipError_t launch_decode(const FwdParams& p, hipStream_t s);

}  // namespace fa
