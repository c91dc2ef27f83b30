// Device-side helpers shared by the builder, prefill and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.hpp"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  // D[m][n] += sum_k A[m][k] B[k][n]; lane l holds A[l%32][8(l/32)..+8], B[8(l/32)..+8][l%32];
  // D: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32.
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Round-to-nearest-even float -> bf16 pair packed into one dword (low = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wave-uniform read of memory no kernel in flight writes (block tables): through the
// constant address space it becomes a scalar load, whose wait does not include the
// wave's pending vector loads and stores.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
  return uniform(*(const __attribute__((address_space(4))) int32_t*)p);
}

// ---------------------------------------------------------------------------------
// Element predicate of the mask menu: postfix program over a one-bit-per-slot stack.
// i is the global query position, j the key position, di/dj their document IDs
// (ignored unless the program holds a document node).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ bool mask_allowed(const MaskProg& p, int i, int j, int di, int dj) {
  uint32_t st = 0;
  int sp = 0;
  for (int t = 0; t < p.n; ++t) {
    const int op = p.op[t];
    const int a = p.arg[t];
    uint32_t v;
    if (op == FA_M_CAUSAL) {
      v = j <= i;
    } else if (op == FA_M_SWA) {
      v = (j <= i) & (i - j < a);
    } else if (op == FA_M_DOC) {
      v = di == dj;
    } else if (op == FA_M_PREFIX) {
      v = (j < a) | (j <= i);
    } else {
      sp -= 2;
      const uint32_t x = (st >> sp) & 1u;
      const uint32_t y = (st >> (sp + 1)) & 1u;
      v = (op == FA_M_AND) ? (x & y) : (x | y);
    }
    st = (st & ~(1u << sp)) | (v << sp);
    ++sp;
  }
  return st & 1u;
}

// ---------------------------------------------------------------------------------
// The same program over a group of up to 32 (query, key) pairs that share a query row
// or a key, one bit per pair.  With one side fixed, every leaf except the document
// test allows one interval of the other side, so a leaf costs one span(lo, hi) -- the
// group's bits of positions in [lo, hi], 0 <= lo, hi <= kPosOpen -- and the document
// leaf the caller's doc_bits (row_leaf: keys of row i; col_leaf: rows of key j).
// And/or act on whole words.  The stack is kMaskStackMax registers shifted on push
// and pop, enough for programs in the host's deeper-first operand order.
// ---------------------------------------------------------------------------------
static_assert(kMaskStackMax == 4, "the word evaluator's stack holds four values");
constexpr int kPosOpen = 0x7ffffffe;   // upper bound of an interval open to the right

template <class Span>
__device__ __forceinline__ uint32_t row_leaf(int op, int a, int i, const Span& span, uint32_t doc_bits) {
  if (op == FA_M_CAUSAL) return span(0, i);                     // j <= i
  if (op == FA_M_SWA) return span(max(i - a + 1, 0), i);        // i - W < j <= i
  if (op == FA_M_PREFIX) return span(0, max(i, a - 1));         // j < P or j <= i
  return doc_bits;
}

template <class Span>
__device__ __forceinline__ uint32_t col_leaf(int op, int a, int j, const Span& span, uint32_t doc_bits) {
  if (op == FA_M_CAUSAL) return span(j, kPosOpen);              // i >= j
  if (op == FA_M_SWA) return span(j, (int)min((int64_t)j + a - 1, (int64_t)kPosOpen));
  if (op == FA_M_PREFIX) return span(j < a ? 0 : j, kPosOpen);  // every row when j < P
  return doc_bits;
}

// leaf(op, arg) -> word of the leaf
template <class Leaf>
__device__ __forceinline__ uint32_t mask_word(const MaskProg& p, const Leaf& leaf) {
  uint32_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll
  for (int t = 0; t < FA_MASK_MAX_NODES; ++t) {
    if (t >= p.n) break;
    const int op = p.op[t];
    if (op == FA_M_AND || op == FA_M_OR) {
      s0 = op == FA_M_AND ? (s0 & s1) : (s0 | s1);
      s1 = s2; s2 = s3;
    } else {
      const uint32_t v = leaf(op, p.arg[t]);
      s3 = s2; s2 = s1; s1 = s0; s0 = v;
    }
  }
  return s0;
}

// ---------------------------------------------------------------------------------
// Score modification in the base-2 domain: returns log2(e) * score_mod(s * scale).
// Order of operations follows the definition: scale, then modify; masking to -inf
// happens afterwards at the call site.
// ---------------------------------------------------------------------------------
struct ScoreCtx {
  float c2;          // scale * log2(e)
  float slope2;      // ALiBi slope of the query head * log2(e)
  const float* tab;  // relative-position row of the query head
  int radius;
  float cap2;        // softcap * log2(e)
  float capk;        // 2 * scale * log2(e) / softcap
};

__device__ __forceinline__ ScoreCtx make_score_ctx(const ScoreParams& sp, float scale, int hq) {
  ScoreCtx c;
  c.c2 = scale * kLog2e;
  c.slope2 = 0.f;
  c.tab = nullptr;
  c.radius = sp.radius;
  c.cap2 = 0.f;
  c.capk = 0.f;
  if (sp.kind == FA_S_ALIBI) c.slope2 = sp.slopes[hq] * kLog2e;
  if (sp.kind == FA_S_RELPOS) c.tab = sp.table + (int64_t)hq * (2 * sp.radius + 1);
  if (sp.kind == FA_S_SOFTCAP) {
    c.cap2 = sp.softcap * kLog2e;
    c.capk = 2.f * scale * kLog2e / sp.softcap;
  }
  return c;
}

template <int SCORE>
__device__ __forceinline__ float score_log2(float s, const ScoreCtx& c, int i_g, int j) {
  if constexpr (SCORE == FA_S_IDENTITY) {
    return s * c.c2;
  } else if constexpr (SCORE == FA_S_ALIBI) {
    return s * c.c2 + c.slope2 * (float)(j - i_g);
  } else if constexpr (SCORE == FA_S_SOFTCAP) {
    // CAP * tanh(x) with tanh x = 1 - 2 / (e^{2x} + 1), e^{2x} from the hardware exp2
    const float u = fast_exp2(s * c.capk);
    return c.cap2 - 2.f * c.cap2 * fast_rcp(u + 1.f);
  } else {
    int rel = i_g - j;
    rel = rel < -c.radius ? -c.radius : (rel > c.radius ? c.radius : rel);
    return s * c.c2 + c.tab[rel + c.radius] * kLog2e;
  }
}

__device__ __forceinline__ const int32_t* doc_row(const DocRef& d, int b) {
  return d.ids ? d.ids + (d.batch == 1 ? 0 : (int64_t)b * d.len) : nullptr;
}

}  // namespace fa
