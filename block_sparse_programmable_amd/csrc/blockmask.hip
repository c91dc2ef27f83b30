// BlockMask builder for gfx950: exact three-state block classification and
// compaction into BCSR rows plus their transposes.
//
// Definitions followed
//   * "FlexAttention: from rules to fused kernels", section 6.3 -- a block is skipped
//     when its allowed edge set E_rc is empty, is full when E_rc is the whole block,
//     partial otherwise; completeness, exclusivity and exactness are required.
//   * same page, section 6.3 ("interval rules avoid quadratic construction") -- for a
//     windowed row i the allowed keys form [max(0, i-W+1), i]; over a query block the
//     union decides candidates and the intersection decides full blocks.  Prefix and
//     document rules also have boundary structure.
//   * same page, sections 2.1-2.2 -- per-row counts and column indices (BCSR), full and
//     partial lists kept apart, transposed query-side index for the backward.
//   * "Causal block geometric pruning", section 5 -- ragged last blocks are clipped to
//     the real sequence end.
//
// Classification uses four values per rule node on a block: T (every in-range pair
// allowed), F (none), M (exactly mixed) and U (not decided by the bounds).  Interval
// leaves (causal, window, prefix) are always decided exactly (T/F/M) from the block's
// row and column ranges; a document leaf is T when one document spans all rows and
// columns, F when the row and column document-ID ranges are disjoint, else U.  And/or
// combine in Kleene fashion (T and x = x, F or x = x, two mixed operands give U).
// Blocks left at U are decided exactly by one wavefront that evaluates every in-range
// pair with ballots (early exit once both an allowed and a disallowed pair are seen).
// No conservative answer is ever emitted.
//
// Launches (all on the caller's stream, no host synchronisation):
//   1. doc_stats   (only with a document rule) doc-ID min/max per query/KV block
//   2. classify    one lane per block, then the wave resolves its undecided blocks
//   3. count       one wave per row and per column: partial/full counts (ballot+popcount)
//   4. scan        one workgroup: exclusive prefix sums of the four count arrays
//   5. scatter     one wave per row and per column: ordered compaction (ballot+mbcnt)
// Nothing uses atomics, so the tables are bit-for-bit deterministic.
#include "device_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr uint8_t kEmpty = 0, kPartial = 1, kFull = 2;
enum : int { VT = 0, VF = 1, VM = 2, VU = 3 };

__device__ __forceinline__ int v_and(int x, int y) {
  if (x == VF || y == VF) return VF;
  if (x == VT) return y;
  if (y == VT) return x;
  return VU;
}
__device__ __forceinline__ int v_or(int x, int y) {
  if (x == VT || y == VT) return VT;
  if (x == VF) return y;
  if (y == VF) return x;
  return VU;
}

struct BlockGeom {
  int64_t a, bb;   // global row range (in range)
  int64_t c0, c1;  // column range (in range)
};

__device__ __forceinline__ BlockGeom geom(const BuildParams& p, int r, int c) {
  BlockGeom g;
  const int64_t r0 = (int64_t)r * p.bq;
  const int64_t r1 = min((int64_t)(r + 1) * p.bq, p.q_len) - 1;
  g.a = r0 + p.q_offset;
  g.bb = r1 + p.q_offset;
  g.c0 = (int64_t)c * p.bk;
  g.c1 = min((int64_t)(c + 1) * p.bk, p.kv_len) - 1;
  return g;
}

__device__ int classify_bounds(const BuildParams& p, const BlockGeom& g, int tb, int r, int c) {
  int st[FA_MASK_MAX_NODES];
  int sp = 0;
  for (int t = 0; t < p.prog.n; ++t) {
    const int op = p.prog.op[t];
    const int64_t a = p.prog.arg[t];
    int v;
    if (op == FA_M_CAUSAL) {
      v = (g.c1 <= g.a) ? VT : (g.c0 > g.bb ? VF : VM);
    } else if (op == FA_M_SWA) {
      if (g.c1 <= g.a && g.c0 >= g.bb - a + 1) v = VT;
      else if (g.c0 > g.bb || g.c1 < g.a - a + 1) v = VF;
      else v = VM;
    } else if (op == FA_M_PREFIX) {
      const int64_t hi_a = max(a - 1, g.a), hi_b = max(a - 1, g.bb);
      v = (g.c1 <= hi_a) ? VT : (g.c0 > hi_b ? VF : VM);
    } else if (op == FA_M_DOC) {
      const int32_t* qs = p.qstat + ((int64_t)tb * p.nqb + r) * 2;
      const int32_t* ks = p.kstat + ((int64_t)tb * p.nkb + c) * 2;
      const int qmin = qs[0], qmax = qs[1], kmin = ks[0], kmax = ks[1];
      if (qmin == qmax && kmin == kmax && qmin == kmin) v = VT;
      else if (qmax < kmin || kmax < qmin) v = VF;
      else v = VU;
    } else {
      sp -= 2;
      const int x = st[sp], y = st[sp + 1];
      if (op == FA_M_AND) {
        v = v_and(x, y);
        if (v == VM && x == VM && y == VM) v = VU;
      } else {
        v = v_or(x, y);
        if (v == VM && x == VM && y == VM) v = VU;
      }
    }
    st[sp++] = v;
  }
  return st[0];
}

// doc-ID min/max per query block (first tB*nqb waves) and per KV block (the rest)
__global__ __launch_bounds__(256) void doc_stats_kernel(BuildParams p) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nq = p.tB * p.nqb;
  const int nk = p.tB * p.nkb;
  if (wave >= nq + nk) return;
  const bool qside = wave < nq;
  const int idx = qside ? wave : wave - nq;
  const int tb = qside ? idx / p.nqb : idx / p.nkb;
  const int blk = qside ? idx - tb * p.nqb : idx - tb * p.nkb;
  const int32_t* d = doc_row(p.doc, tb);
  int64_t lo, hi;
  if (qside) {
    lo = (int64_t)blk * p.bq;
    hi = min((int64_t)(blk + 1) * p.bq, p.q_len);
    lo += p.q_offset;
    hi += p.q_offset;
  } else {
    lo = (int64_t)blk * p.bk;
    hi = min((int64_t)(blk + 1) * p.bk, p.kv_len);
  }
  int mn = 0x7fffffff, mx = (int)0x80000000;
  for (int64_t x = lo + lane; x < hi; x += 64) {
    const int v = d[x];
    mn = min(mn, v);
    mx = max(mx, v);
  }
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, __shfl_xor(mn, off));
    mx = max(mx, __shfl_xor(mx, off));
  }
  if (lane == 0) {
    int32_t* out = (qside ? p.qstat : p.kstat) + (int64_t)idx * 2;
    out[0] = mn;
    out[1] = mx;
  }
}

__global__ __launch_bounds__(256) void classify_kernel(BuildParams p) {
  const int64_t total = (int64_t)p.tB * p.nqb * p.nkb;
  const int64_t wave_base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  const int lane = threadIdx.x & 63;
  if (wave_base >= total) return;
  const int64_t id = wave_base + lane;
  int val = VF;
  int tb = 0, r = 0, c = 0;
  const bool valid = id < total;
  if (valid) {
    tb = (int)(id / ((int64_t)p.nqb * p.nkb));
    const int64_t rem = id - (int64_t)tb * p.nqb * p.nkb;
    r = (int)(rem / p.nkb);
    c = (int)(rem - (int64_t)r * p.nkb);
    val = classify_bounds(p, geom(p, r, c), tb, r, c);
    if (val != VU) p.grid[id] = val == VT ? kFull : (val == VF ? kEmpty : kPartial);
  }
  // exact evaluation of undecided blocks, one block at a time with the whole wave
  uint64_t pending = __ballot(valid && val == VU);
  while (pending) {
    const int src = __builtin_ctzll(pending);
    pending &= pending - 1;
    const int ub = __shfl(tb, src), ur = __shfl(r, src), uc = __shfl(c, src);
    const BlockGeom g = geom(p, ur, uc);
    const int32_t* d = doc_row(p.doc, ub);
    const int ncols = (int)(g.c1 - g.c0 + 1);
    const int j0 = (int)g.c0 + lane;
    const int j1 = j0 + 64;
    const bool ok0 = lane < ncols, ok1 = lane + 64 < ncols;
    const int dj0 = (p.prog.has_doc && ok0) ? d[j0] : 0;
    const int dj1 = (p.prog.has_doc && ok1) ? d[j1] : 0;
    bool seen_t = false, seen_f = false;
    for (int64_t i = g.a; i <= g.bb; ++i) {
      const int ii = (int)i;
      const int di = p.prog.has_doc ? d[ii] : 0;
      const bool m0 = ok0 && mask_allowed(p.prog, ii, j0, di, dj0);
      const bool m1 = ok1 && mask_allowed(p.prog, ii, j1, di, dj1);
      seen_t = seen_t || (__ballot(m0 || m1) != 0);
      seen_f = seen_f || (__ballot((ok0 && !m0) || (ok1 && !m1)) != 0);
      if (seen_t && seen_f) break;
    }
    if (lane == 0) {
      const int64_t uid = ((int64_t)ub * p.nqb + ur) * p.nkb + uc;
      p.grid[uid] = seen_t ? (seen_f ? kPartial : kFull) : kEmpty;
    }
  }
}

// one wave per kv-side row (tb, r) and per q-side column (tb, c); writes counts for
// every replicated head
__global__ __launch_bounds__(256) void count_kernel(BuildParams p) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nr = p.tB * p.nqb;
  const int nc = p.tB * p.nkb;
  if (wave >= nr + nc) return;
  const bool rowside = wave < nr;
  const int idx = rowside ? wave : wave - nr;
  const int n = rowside ? p.nkb : p.nqb;
  const int tb = rowside ? idx / p.nqb : idx / p.nkb;
  const int k = rowside ? idx - tb * p.nqb : idx - tb * p.nkb;
  const uint8_t* g = p.grid + (int64_t)tb * p.nqb * p.nkb;
  int np = 0, nf = 0;
  for (int x0 = 0; x0 < n; x0 += 64) {
    const int x = x0 + lane;
    uint8_t v = kEmpty;
    if (x < n) v = rowside ? g[(int64_t)k * p.nkb + x] : g[(int64_t)x * p.nkb + k];
    np += __popcll(__ballot(v == kPartial));
    nf += __popcll(__ballot(v == kFull));
  }
  if (lane < p.tH) {
    for (int h = lane; h < p.tH; h += 64) {
      if (rowside) {
        const int64_t rr = ((int64_t)tb * p.tH + h) * p.nqb + k;
        p.kv_num[rr] = np;
        p.full_kv_num[rr] = nf;
      } else {
        const int64_t cc = ((int64_t)tb * p.tH + h) * p.nkb + k;
        p.q_num[cc] = np;
        p.full_q_num[cc] = nf;
      }
    }
  }
}

// single workgroup: exclusive scans of the four count arrays
__global__ __launch_bounds__(1024) void scan_kernel(BuildParams p) {
  __shared__ int32_t warp_sums[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int which = 0; which < 4; ++which) {
    const int32_t* num = which == 0 ? p.kv_num : which == 1 ? p.full_kv_num : which == 2 ? p.q_num : p.full_q_num;
    int32_t* ptr = which == 0 ? p.kv_ptr : which == 1 ? p.full_kv_ptr : which == 2 ? p.q_ptr : p.full_q_ptr;
    const int64_t n = (which < 2) ? (int64_t)p.tB * p.tH * p.nqb : (int64_t)p.tB * p.tH * p.nkb;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int64_t base = 0; base < n; base += 1024) {
      const int64_t x = base + tid;
      const int v = x < n ? num[x] : 0;
      // inclusive scan within the wave
      int s = v;
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(s, off);
        if (lane >= off) s += y;
      }
      if (lane == 63) warp_sums[wv] = s;
      __syncthreads();
      int wprefix = 0;
      for (int q = 0; q < wv; ++q) wprefix += warp_sums[q];
      const int carry = carry_s;
      if (x < n) ptr[x] = carry + wprefix + s - v;
      __syncthreads();
      if (tid == 1023) carry_s = carry + wprefix + s;
      __syncthreads();
    }
    if (tid == 0) ptr[n] = carry_s;
    __syncthreads();
  }
}

// ordered compaction, one wave per (tb, h, row) and per (tb, h, column)
__global__ __launch_bounds__(256) void scatter_kernel(BuildParams p) {
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t nr = (int64_t)p.tB * p.tH * p.nqb;
  const int64_t nc = (int64_t)p.tB * p.tH * p.nkb;
  if (wave >= nr + nc) return;
  const bool rowside = wave < nr;
  const int64_t idx = rowside ? wave : wave - nr;
  const int per = rowside ? p.nqb : p.nkb;
  const int64_t bh = idx / per;
  const int k = (int)(idx - bh * per);
  const int tb = (int)(bh / p.tH);
  const int n = rowside ? p.nkb : p.nqb;
  const uint8_t* g = p.grid + (int64_t)tb * p.nqb * p.nkb;
  int32_t* pout = rowside ? p.kv_idx + p.kv_ptr[idx] : p.q_idx + p.q_ptr[idx];
  int32_t* fout = rowside ? p.full_kv_idx + p.full_kv_ptr[idx] : p.full_q_idx + p.full_q_ptr[idx];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int x0 = 0; x0 < n; x0 += 64) {
    const int x = x0 + lane;
    uint8_t v = kEmpty;
    if (x < n) v = rowside ? g[(int64_t)k * p.nkb + x] : g[(int64_t)x * p.nkb + k];
    const uint64_t bp = __ballot(v == kPartial);
    const uint64_t bf = __ballot(v == kFull);
    if (v == kPartial) pout[__popcll(bp & below)] = x;
    if (v == kFull) fout[__popcll(bf & below)] = x;
    pout += __popcll(bp);
    fout += __popcll(bf);
  }
}

inline unsigned waves_to_blocks(int64_t waves) { return (unsigned)((waves + 3) / 4); }

}  // namespace

size_t build_workspace_bytes(int64_t tB, int64_t nqb, int64_t nkb) {
  const size_t grid = (size_t)(tB * nqb * nkb + 255) & ~(size_t)255;
  const size_t stats = (size_t)tB * (nqb + nkb) * 2 * sizeof(int32_t);
  return grid + ((stats + 255) & ~(size_t)255);
}

hipError_t launch_build(const BuildParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.tB * p.nqb * p.nkb;
  if (total == 0) return hipSuccess;
  if (p.prog.has_doc) {
    hipLaunchKernelGGL(doc_stats_kernel, dim3(waves_to_blocks((int64_t)p.tB * (p.nqb + p.nkb))), dim3(256), 0, s, p);
  }
  hipLaunchKernelGGL(classify_kernel, dim3(waves_to_blocks((total + 63) / 64)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(count_kernel, dim3(waves_to_blocks((int64_t)p.tB * (p.nqb + p.nkb))), dim3(256), 0, s, p);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(scatter_kernel, dim3(waves_to_blocks((int64_t)p.tB * p.tH * (p.nqb + p.nkb))), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
