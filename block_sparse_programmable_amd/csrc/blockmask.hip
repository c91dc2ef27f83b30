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
// Grids of at most 16384 blocks are built by one workgroup in a single launch with all
// intermediates in LDS.  Larger grids use five launches (all on the caller's stream,
// no host synchronisation):
//   1. doc_stats   (only with a document rule) doc-ID min/max per query/KV block
//   2. classify    one lane per block, then the wave resolves its undecided blocks
//   3. count       one wave per row and per column: partial/full counts (ballot+popcount)
//   4. scan        one workgroup per count array: exclusive prefix sums
//   5. scatter     one wave per row and per column: ordered compaction (ballot+mbcnt)
// No output position depends on an atomic or on scheduling order (the single-workgroup
// path collects undecided blocks in an LDS list whose order does not matter), so the
// tables are bit-for-bit deterministic.
#include "device_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

// wave-wide exclusive prefix sum (DPP), from the device library that also provides the
// wave reductions used below
extern "C" __device__ int __ockl_wfscan_add_i32(int, bool);

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

// Document part from the per-block ID ranges.  When the IDs are non-decreasing over
// every position either side reads (docs_sorted), the IDs present in a block are all the
// present IDs between its min and max, so two blocks share an ID iff their ranges
// overlap: overlapping ranges that are not one common ID make a known partial block.
__device__ __forceinline__ int classify_doc(const int32_t* qs, const int32_t* ks, bool docs_sorted) {
  const int qmin = qs[0], qmax = qs[1], kmin = ks[0], kmax = ks[1];
  if (qmin == qmax && kmin == kmax && qmin == kmin) return VT;
  if (qmax < kmin || kmax < qmin) return VF;
  return docs_sorted ? VM : VU;
}

// And-only programs (interval form): the allowed keys of row i are [lo(i), hi(i)] with
// both ends non-decreasing in i and lo(i) <= i <= hi(i), so the block is FULL iff
// lo(last row) <= c0 and hi(first row) >= c1, and EMPTY iff no row reaches the block:
// the first row i1 with hi(i1) >= c0 has the smallest lo among the rows that do, so the
// block is empty iff there is no such row or lo(i1) > c1.  Otherwise it is partial.
__device__ int classify_interval(const BuildParams& p, const BlockGeom& g, const int32_t* qs, const int32_t* ks,
                                 bool docs_sorted) {
  const MaskProg& m = p.prog;
  auto lo_of = [&](int64_t i) -> int64_t { return m.wmin > 0 ? max((int64_t)0, i - m.wmin + 1) : (int64_t)0; };
  auto hi_of = [&](int64_t i) -> int64_t {
    return m.hi_self ? i : (m.pmin >= 0 ? max((int64_t)m.pmin - 1, i) : (int64_t)0x7fffffffffffffffLL);
  };
  int v;
  if (lo_of(g.bb) <= g.c0 && hi_of(g.a) >= g.c1) {
    v = VT;
  } else {
    int64_t i1;
    if (m.hi_self) i1 = max(g.a, g.c0);
    else if (m.pmin >= 0) i1 = (int64_t)m.pmin - 1 >= g.c0 ? g.a : max(g.a, g.c0);
    else i1 = g.a;
    v = (i1 > g.bb || lo_of(i1) > g.c1) ? VF : VM;
  }
  if (m.has_doc) v = v_and(v, classify_doc(qs, ks, docs_sorted));
  return v;
}

// classify_interval for positions that fit in 32 bits, with the row block's quantities
// (first row a, last row bb, lo(bb), hi(a)) computed once per row by the caller
__device__ __forceinline__ int classify_interval32(const MaskProg& m, int a, int bb, int lo_bb, int hi_a, int c0,
                                                   int c1, const int32_t* qs, const int32_t* ks, bool docs_sorted) {
  int v;
  if (lo_bb <= c0 && hi_a >= c1) {
    v = VT;
  } else {
    const int i1 = m.hi_self ? max(a, c0) : (m.pmin >= 0 ? (m.pmin - 1 >= c0 ? a : max(a, c0)) : a);
    const int lo_i1 = m.wmin > 0 ? max(0, i1 - m.wmin + 1) : 0;
    v = (i1 > bb || lo_i1 > c1) ? VF : VM;
  }
  if (m.has_doc) v = v_and(v, classify_doc(qs, ks, docs_sorted));
  return v;
}

__device__ int classify_bounds(const BuildParams& p, const BlockGeom& g, const int32_t* qs, const int32_t* ks,
                               bool docs_sorted = false) {
  if (p.prog.mk != MK_GENERIC) return classify_interval(p, g, qs, ks, docs_sorted);
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
      v = classify_doc(qs, ks, docs_sorted);
    } else {
      sp -= 2;
      const int x = st[sp], y = st[sp + 1];
      v = (op == FA_M_AND) ? v_and(x, y) : v_or(x, y);
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

// Exact class of one block, decided by the whole wave.
//
// Fast form (and-only programs whose KV block holds non-decreasing document IDs in at
// most eight runs): the keys of the block that share row i's document are one
// contiguous range, read off the runs (start column and ID, wave-uniform); with the
// row's compiled key interval that gives the row's allowed keys as one interval, so each
// lane decides two rows outright ("FlexAttention: from rules to fused kernels",
// section 6.3: document rules have boundary structure too).
//
// General form: lanes cover the block's columns, rows are walked in order with their
// document IDs held in registers and broadcast by readlane; stops as soon as both an
// allowed and a disallowed in-range pair have been seen.  And-only programs test each
// pair against the row's compiled key interval plus the document compare; programs
// with an or-node use the interpreter.
// document IDs of a block's columns (j0, j0 + 64) and rows (a, a + 64) for this lane
struct BlockDocs {
  int dj0, dj1, dr0, dr1;
};

__device__ __forceinline__ BlockDocs load_block_docs(const BuildParams& p, int tb, int r, int c, int lane) {
  BlockDocs bd = {0, 0, 0, 0};
  if (!p.prog.has_doc) return bd;
  const BlockGeom g = geom(p, r, c);
  const int32_t* d = doc_row(p.doc, tb);
  const int nrows = (int)(g.bb - g.a + 1);
  const int ncols = (int)(g.c1 - g.c0 + 1);
  if (lane < ncols) bd.dj0 = d[g.c0 + lane];
  if (lane + 64 < ncols) bd.dj1 = d[g.c0 + 64 + lane];
  if (lane < nrows) bd.dr0 = d[g.a + lane];
  if (lane + 64 < nrows) bd.dr1 = d[g.a + 64 + lane];
  return bd;
}

__device__ uint8_t exact_block(const BuildParams& p, int tb, int r, int c, int lane, const BlockDocs& bd) {
  const BlockGeom g = geom(p, r, c);
  const int nrows = (int)(g.bb - g.a + 1);
  const int ncols = (int)(g.c1 - g.c0 + 1);
  const int a = (int)g.a;
  const int j0 = (int)g.c0 + lane;
  const int j1 = j0 + 64;
  const bool ok0 = lane < ncols, ok1 = lane + 64 < ncols;
  const int dj0 = bd.dj0, dj1 = bd.dj1, dr0 = bd.dr0, dr1 = bd.dr1;
  const bool interval_form = p.prog.mk != MK_GENERIC;
  if (interval_form && p.prog.has_doc) {
    // the block's columns as runs of equal document IDs: a run starts where the ID
    // differs from the previous column; IDs must not decrease across the block
    const int last0 = __shfl(dj0, 63);
    const int prev0 = __shfl(dj0, lane > 0 ? lane - 1 : 0);
    const int prev1 = lane > 0 ? __shfl(dj1, lane - 1) : last0;
    const bool desc = (ok0 && lane > 0 && dj0 < prev0) || (ok1 && dj1 < prev1);
    uint64_t m0 = __ballot(ok0 && (lane == 0 || dj0 != prev0));
    uint64_t m1 = __ballot(ok1 && dj1 != prev1);
    constexpr int kRuns = 8;
    if (__ballot(desc) == 0 && __popcll(m0) + __popcll(m1) <= kRuns) {
      // run k: first column rs[k], ID rv[k] (wave-uniform); unused runs keep rs = ncols
      int rs[kRuns], rv[kRuns];
#pragma unroll
      for (int k = 0; k < kRuns; ++k) {
        rs[k] = ncols;
        rv[k] = 0x7fffffff;
        if (m0) {
          const int pos = __builtin_ctzll(m0);
          m0 &= m0 - 1;
          rs[k] = pos;
          rv[k] = __builtin_amdgcn_readlane(dj0, pos);
        } else if (m1) {
          const int pos = __builtin_ctzll(m1);
          m1 &= m1 - 1;
          rs[k] = 64 + pos;
          rv[k] = __builtin_amdgcn_readlane(dj1, pos);
        }
      }
      bool not_full = false, not_empty = false;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ri = lane + 64 * q;
        if (ri < nrows) {
          const int ii = a + ri;
          const int di = q == 0 ? dr0 : dr1;
          // columns with ID == di: [first run with ID >= di, first run with ID > di)
          int lb = ncols, ub = ncols;
#pragma unroll
          for (int k = kRuns - 1; k >= 0; --k) {
            if (rv[k] >= di) lb = rs[k];
            if (rv[k] > di) ub = rs[k];
          }
          int lo = p.prog.wmin > 0 ? max(0, ii - p.prog.wmin + 1) : 0;
          int hi = p.prog.hi_self ? ii : (p.prog.pmin >= 0 ? max(p.prog.pmin - 1, ii) : 0x7fffffff);
          const int c0 = (int)g.c0, c1 = (int)g.c1;
          lo = max(lo, c0 + lb);
          hi = min(hi, c0 + ub - 1);
          const bool full = lo <= c0 && hi >= c1;
          const bool empty = max(lo, c0) > min(hi, c1);
          not_full = not_full || !full;
          not_empty = not_empty || !empty;
        }
      }
      const bool all_full = __ballot(not_full) == 0;
      const bool all_empty = __ballot(not_empty) == 0;
      return all_full ? kFull : (all_empty ? kEmpty : kPartial);
    }
  }
  bool seen_t = false, seen_f = false;
  for (int ri = 0; ri < nrows; ++ri) {
    const int ii = a + ri;
    const int di = p.prog.has_doc ? __builtin_amdgcn_readlane(ri < 64 ? dr0 : dr1, ri & 63) : 0;
    bool m0, m1;
    if (interval_form) {
      // allowed keys of row ii: [lo, hi] (uniform across the wave)
      const int lo = p.prog.wmin > 0 ? max(0, ii - p.prog.wmin + 1) : 0;
      const int hi = p.prog.hi_self ? ii : (p.prog.pmin >= 0 ? max(p.prog.pmin - 1, ii) : 0x7fffffff);
      m0 = ok0 && j0 >= lo && j0 <= hi && dj0 == di;
      m1 = ok1 && j1 >= lo && j1 <= hi && dj1 == di;
    } else {
      m0 = ok0 && mask_allowed(p.prog, ii, j0, di, dj0);
      m1 = ok1 && mask_allowed(p.prog, ii, j1, di, dj1);
    }
    seen_t = seen_t || (__ballot(m0 || m1) != 0);
    seen_f = seen_f || (__ballot((ok0 && !m0) || (ok1 && !m1)) != 0);
    if (seen_t && seen_f) break;
  }
  return seen_t ? (seen_f ? kPartial : kFull) : kEmpty;
}

constexpr int kClassifyPerWave = 16;   // blocks decided per wave (fast path on 16 lanes)

__global__ __launch_bounds__(256) void classify_kernel(BuildParams p) {
  const int64_t total = (int64_t)p.tB * p.nqb * p.nkb;
  const int64_t wave_base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kClassifyPerWave;
  const int lane = threadIdx.x & 63;
  if (wave_base >= total) return;
  const int64_t id = wave_base + lane;
  int val = VF;
  int tb = 0, r = 0, c = 0;
  const bool valid = lane < kClassifyPerWave && id < total;
  if (valid) {
    tb = (int)(id / ((int64_t)p.nqb * p.nkb));
    const int64_t rem = id - (int64_t)tb * p.nqb * p.nkb;
    r = (int)(rem / p.nkb);
    c = (int)(rem - (int64_t)r * p.nkb);
    val = classify_bounds(p, geom(p, r, c), p.qstat + ((int64_t)tb * p.nqb + r) * 2,
                          p.kstat + ((int64_t)tb * p.nkb + c) * 2);
    if (val != VU) p.grid[id] = val == VT ? kFull : (val == VF ? kEmpty : kPartial);
  }
  // exact evaluation of undecided blocks, one block at a time with the whole wave
  uint64_t pending = __ballot(valid && val == VU);
  while (pending) {
    const int src = __builtin_ctzll(pending);
    pending &= pending - 1;
    const int ub = __shfl(tb, src), ur = __shfl(r, src), uc = __shfl(c, src);
    const uint8_t cls = exact_block(p, ub, ur, uc, lane, load_block_docs(p, ub, ur, uc, lane));
    if (lane == 0) p.grid[((int64_t)ub * p.nqb + ur) * p.nkb + uc] = cls;
  }
}

// one wave per kv-side row (tb, r) and per q-side column (tb, c); writes counts for
// every replicated head
__global__ __launch_bounds__(256) void count_kernel(BuildParams p) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nr = p.tB * p.nqb;
  const int nc = p.q_num ? p.tB * p.nkb : 0;   // query side not requested: rows only
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

// exclusive scans of the four count arrays, one workgroup per array (blockIdx.x), each
// thread taking four consecutive counts per pass (DPP wave scans, wave totals in LDS)
__global__ __launch_bounds__(1024) void scan_kernel(BuildParams p) {
  __shared__ int32_t wave_sums[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
  const int which = blockIdx.x;
  const int32_t* num = which == 0 ? p.kv_num : which == 1 ? p.full_kv_num : which == 2 ? p.q_num : p.full_q_num;
  int32_t* ptr = which == 0 ? p.kv_ptr : which == 1 ? p.full_kv_ptr : which == 2 ? p.q_ptr : p.full_q_ptr;
  if (num == nullptr) return;   // query side not requested (kernel argument: uniform)
  const int64_t n = (which < 2) ? (int64_t)p.tB * p.tH * p.nqb : (int64_t)p.tB * p.tH * p.nkb;
  int carry = 0;
  for (int64_t base = 0; base < n; base += 4096) {
    const int64_t x0 = base + 4 * (int64_t)tid;
    int v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x0 + e < n ? num[x0 + e] : 0;
    const int t = v[0] + v[1] + v[2] + v[3];
    const int excl = __ockl_wfscan_add_i32(t, false);
    if (lane == 63) wave_sums[wv] = excl + t;
    __syncthreads();
    int wprefix = 0, total = 0;
    for (int q = 0; q < 16; ++q) {
      const int ws = wave_sums[q];
      wprefix += q < wv ? ws : 0;
      total += ws;
    }
    int run = carry + wprefix + excl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (x0 + e < n) ptr[x0 + e] = run;
      run += v[e];
    }
    carry += total;
    __syncthreads();   // wave_sums is rewritten by the next pass
  }
  if (tid == 0) ptr[n] = carry;
}

// ordered compaction, one wave per (tb, h, row) and per (tb, h, column)
__global__ __launch_bounds__(256) void scatter_kernel(BuildParams p) {
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t nr = (int64_t)p.tB * p.tH * p.nqb;
  const int64_t nc = p.q_num ? (int64_t)p.tB * p.tH * p.nkb : 0;
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

// ---------------------------------------------------------------------------------
// Small grids: the whole build in one workgroup of 16 waves, intermediates in LDS.
// Same phases and the same per-block decisions as the multi-launch path.
// ---------------------------------------------------------------------------------
constexpr int kSmallMaxBlocks = 16384;  // tB * NQB * NKB
constexpr int kSmallMaxLines = 2048;    // tB * (NQB + NKB)
constexpr int kSmallMaxTB = 64;
constexpr int kOrderInlineRows = 256;   // groups of at most this many rows are ranked in place

// the work-order entry of row r of table group tb, by one wave: its rank among the
// group's rows by descending length, ties by descending index (the lanes count 64 rows
// at a time with a ballot), written for every head of the group
template <class LenF>
__device__ __forceinline__ void rank_row(const BuildParams& p, int tb, int r, int lane, LenF len_of) {
  const int len = len_of(r);
  int rank = 0;
  for (int y0 = 0; y0 < p.nqb; y0 += 512) {   // eight reads in flight, then their ballots
    int ly[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int y = y0 + 64 * u + lane;
      ly[u] = y < p.nqb ? len_of(y) : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int y = y0 + 64 * u + lane;
      rank += __popcll(__ballot(ly[u] > len || (ly[u] == len && y > r)));
    }
  }
  for (int h = lane; h < p.tH; h += 64) p.order[((int64_t)tb * p.tH + h) * p.nqb + rank] = r;
}

// phases 4-6 of the one-workgroup build, shared with the row slicer: partial/full
// counts (skipped when `counted`: cnt_s already holds them), prefix sums and ordered
// compaction of an LDS class grid [tB][nqb][nkb] into the table arrays, every row and
// column repeated for the tH heads of its tb.  The query-side arrays are written only
// when p.q_num is set.
__device__ void compact_small(const BuildParams& p, const uint8_t* grid_s, int32_t* cnt_s, int32_t* pre_s,
                              int32_t* tot_s, int32_t* cum_s, bool counted) {
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
  const int nq = p.tB * p.nqb, nl = nq + p.tB * p.nkb;
  const bool qout = p.q_num != nullptr;
  // phase 4: partial / full counts per row (tb, r) and per column (tb, c).  Every line
  // of a side has the same length; a side of short lines (at most kShort entries, e.g.
  // the query side of a decode grid) takes one thread per line, the other one wave per
  // line (ballot counts).  Lines are [rows | columns], so each kind is one range.
  constexpr int kShort = 8;
  const bool rows_long = p.nkb > kShort, cols_long = p.nqb > kShort;
  const int lw0 = rows_long ? 0 : nq, lw1 = cols_long ? nl : nq;   // long lines
  const int ls0 = rows_long ? nq : 0, ls1 = cols_long ? nq : nl;   // short lines
  auto line_geom = [&](int line, int& tb, int& k, int& n, bool& rowside) {
    rowside = line < nq;
    const int idx = rowside ? line : line - nq;
    tb = p.tB == 1 ? 0 : (rowside ? idx / p.nqb : idx / p.nkb);   // (no divide for one group)
    k = rowside ? idx - tb * p.nqb : idx - tb * p.nkb;
    n = rowside ? p.nkb : p.nqb;
  };
  auto entry = [&](const uint8_t* g, bool rowside, int k, int x) -> uint8_t {
    return rowside ? g[k * p.nkb + x] : g[x * p.nkb + k];
  };
  for (int line = lw0 + wv; line < (counted ? lw0 : lw1); line += 16) {
    int tb, k, n;
    bool rowside;
    line_geom(line, tb, k, n, rowside);
    const uint8_t* g = grid_s + tb * p.nqb * p.nkb;
    int np = 0, nf = 0;
    for (int x0 = 0; x0 < n; x0 += 64) {
      const int x = x0 + lane;
      const uint8_t v = x < n ? entry(g, rowside, k, x) : kEmpty;
      np += __popcll(__ballot(v == kPartial));
      nf += __popcll(__ballot(v == kFull));
    }
    if (lane == 0) {
      cnt_s[2 * line] = np;
      cnt_s[2 * line + 1] = nf;
    }
  }
  for (int line = ls0 + tid; line < (counted ? ls0 : ls1); line += 1024) {
    int tb, k, n;
    bool rowside;
    line_geom(line, tb, k, n, rowside);
    const uint8_t* g = grid_s + tb * p.nqb * p.nkb;
    int np = 0, nf = 0;
    for (int x = 0; x < n; ++x) {
      const uint8_t v = entry(g, rowside, k, x);
      np += v == kPartial;
      nf += v == kFull;
    }
    cnt_s[2 * line] = np;
    cnt_s[2 * line + 1] = nf;
  }
  __syncthreads();

  // phase 5: exclusive prefix within each tb; one wave per (tb, side, kind) sequence
  for (int sq = wv; sq < 4 * p.tB; sq += 16) {
    const int tb = sq >> 2, side = (sq >> 1) & 1, kind = sq & 1;
    const int n = side == 0 ? p.nqb : p.nkb;
    const int first = side == 0 ? tb * p.nqb : nq + tb * p.nkb;
    int carry = 0;
    for (int x0 = 0; x0 < n; x0 += 64) {
      const int x = x0 + lane;
      const int v = x < n ? cnt_s[2 * (first + x) + kind] : 0;
      const int excl = __ockl_wfscan_add_i32(v, false);   // DPP wave scan
      if (x < n) pre_s[2 * (first + x) + kind] = carry + excl;
      carry += __builtin_amdgcn_readlane(excl + v, 63);
    }
    if (lane == 0) tot_s[4 * tb + 2 * side + kind] = carry;
  }
  __syncthreads();
  if (tid < 4) {
    int acc = 0;
    for (int tb = 0; tb < p.tB; ++tb) {
      cum_s[4 * tb + tid] = acc;
      acc += p.tH * tot_s[4 * tb + tid];
    }
    cum_s[4 * p.tB + tid] = acc;
  }
  __syncthreads();

  // work order (when asked for and the groups are short), as order_kernel writes it
  if (p.order && p.nqb <= kOrderInlineRows) {
    for (int x = wv; x < nq; x += 16) {
      const int tb = p.tB == 1 ? 0 : x / p.nqb;
      const int32_t* c = cnt_s + 2 * tb * p.nqb;
      rank_row(p, tb, x - tb * p.nqb, lane, [&](int y) { return c[2 * y] + c[2 * y + 1]; });
    }
  }

  // phase 6: counts and pointers for every replicated head, then ordered scatter
  const int rows = p.tB * p.tH * p.nqb, cols = p.tB * p.tH * p.nkb;
  for (int x = tid; x < rows + (qout ? cols : 0); x += 1024) {
    const bool rowside = x < rows;
    const int idx = rowside ? x : x - rows;
    const int per = rowside ? p.nqb : p.nkb;
    const int bh = p.tB * p.tH == 1 ? 0 : idx / per, k = idx - bh * per;
    const int tb = p.tH == 1 ? bh : bh / p.tH, h = bh - tb * p.tH;
    const int line = rowside ? tb * p.nqb + k : nq + tb * p.nkb + k;
    const int side = rowside ? 0 : 1;
    const int np_ = cnt_s[2 * line], nf_ = cnt_s[2 * line + 1];
    const int pp = cum_s[4 * tb + 2 * side] + h * tot_s[4 * tb + 2 * side] + pre_s[2 * line];
    const int pf = cum_s[4 * tb + 2 * side + 1] + h * tot_s[4 * tb + 2 * side + 1] + pre_s[2 * line + 1];
    if (rowside) {
      p.kv_num[idx] = np_;
      p.kv_ptr[idx] = pp;
      p.full_kv_num[idx] = nf_;
      p.full_kv_ptr[idx] = pf;
    } else {
      p.q_num[idx] = np_;
      p.q_ptr[idx] = pp;
      p.full_q_num[idx] = nf_;
      p.full_q_ptr[idx] = pf;
    }
  }
  if (tid == 0) {
    p.kv_ptr[rows] = cum_s[4 * p.tB + 0];
    p.full_kv_ptr[rows] = cum_s[4 * p.tB + 1];
    if (qout) {
      p.q_ptr[cols] = cum_s[4 * p.tB + 2];
      p.full_q_ptr[cols] = cum_s[4 * p.tB + 3];
    }
  }
  // ordered scatter, per base line and then for every replicated head (head h of tb
  // starts h * tot after head 0): long lines one wave each (ballot compaction), short
  // lines one thread each
  auto line_out = [&](int line, bool rowside, int tb, int& pp0, int& pf0, int& tp, int& tf) {
    const int side = rowside ? 0 : 1;
    tp = tot_s[4 * tb + 2 * side];
    tf = tot_s[4 * tb + 2 * side + 1];
    pp0 = cum_s[4 * tb + 2 * side] + pre_s[2 * line];
    pf0 = cum_s[4 * tb + 2 * side + 1] + pre_s[2 * line + 1];
  };
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int lw1o = qout ? lw1 : min(lw1, nq), ls1o = qout ? ls1 : min(ls1, nq);
  for (int line = lw0 + wv; line < lw1o; line += 16) {
    int tb, k, n, pp0, pf0, tp, tf;
    bool rowside;
    line_geom(line, tb, k, n, rowside);
    line_out(line, rowside, tb, pp0, pf0, tp, tf);
    int32_t* pidx = rowside ? p.kv_idx : p.q_idx;
    int32_t* fidx = rowside ? p.full_kv_idx : p.full_q_idx;
    const uint8_t* g = grid_s + tb * p.nqb * p.nkb;
    for (int x0 = 0; x0 < n; x0 += 64) {
      const int y = x0 + lane;
      const uint8_t v = y < n ? entry(g, rowside, k, y) : kEmpty;
      const uint64_t bp = __ballot(v == kPartial);
      const uint64_t bf = __ballot(v == kFull);
      const int ip = pp0 + __popcll(bp & below), jf = pf0 + __popcll(bf & below);
      for (int h = 0; h < p.tH; ++h) {
        if (v == kPartial) pidx[ip + h * tp] = y;
        if (v == kFull) fidx[jf + h * tf] = y;
      }
      pp0 += __popcll(bp);
      pf0 += __popcll(bf);
    }
  }
  for (int line = ls0 + tid; line < ls1o; line += 1024) {
    int tb, k, n, pp0, pf0, tp, tf;
    bool rowside;
    line_geom(line, tb, k, n, rowside);
    line_out(line, rowside, tb, pp0, pf0, tp, tf);
    int32_t* pidx = rowside ? p.kv_idx : p.q_idx;
    int32_t* fidx = rowside ? p.full_kv_idx : p.full_q_idx;
    const uint8_t* g = grid_s + tb * p.nqb * p.nkb;
    for (int y = 0; y < n; ++y) {
      const uint8_t v = entry(g, rowside, k, y);
      for (int h = 0; h < p.tH; ++h) {
        if (v == kPartial) pidx[pp0 + h * tp] = y;
        if (v == kFull) fidx[pf0 + h * tf] = y;
      }
      pp0 += v == kPartial;
      pf0 += v == kFull;
    }
  }
}

// Document-ID ranges per query block and per KV block by reduction, for IDs that are not
// sorted (the general case of phase 1), and the same order test as doc_ends.  A wave
// takes eight lines at a time (at most 128 IDs each: two per lane, plus the ID after each
// for the order test) and issues all their loads before reducing, so the memory latency
// is paid once per eight lines; the reductions are wave-wide DPP reductions.
__device__ void doc_ranges(const BuildParams& p, int32_t* stat_s, int32_t* unsorted_s) {
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
  const int nq = p.tB * p.nqb, nl = nq + p.tB * p.nkb;
  {
    constexpr int G = 8;
    for (int l0 = wv * G; l0 < nl; l0 += 16 * G) {
      int v[G][2];
      bool in[G][2], inn[G][2];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int line = l0 + u;
        int64_t lo = 0, hi = 1;   // lines past the end read ID 0 of batch 0 and use nothing
        const int32_t* d = doc_row(p.doc, 0);
        if (line < nl) {
          const bool qside = line < nq;
          const int idx = qside ? line : line - nq;
          const int tb = qside ? idx / p.nqb : idx / p.nkb;
          const int blk = qside ? idx - tb * p.nqb : idx - tb * p.nkb;
          d = doc_row(p.doc, tb);
          if (qside) {
            lo = (int64_t)blk * p.bq + p.q_offset;
            hi = min((int64_t)(blk + 1) * p.bq, p.q_len) + p.q_offset;
          } else {
            lo = (int64_t)blk * p.bk;
            hi = min((int64_t)(blk + 1) * p.bk, p.kv_len);
          }
        }
        // unconditional loads at clamped positions keep all of them in flight at once
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t x = lo + lane + 64 * h;
          in[u][h] = line < nl && x < hi;
          inn[u][h] = line < nl && x + 1 < hi;
          v[u][h] = d[min(x, hi - 1)];
        }
      }
      bool any_desc = false;
#pragma unroll
      for (int u = 0; u < G; ++u) {
        // the ID one position on: the next lane's (DPP wave shift left by one lane); for
        // lane 63 of the first half, lane 0 of the second
        const int nx0 = __builtin_amdgcn_update_dpp(__builtin_amdgcn_readlane(v[u][1], 0), v[u][0], 0x130, 0xf, 0xf, false);
        const int nx1 = __builtin_amdgcn_update_dpp(v[u][1], v[u][1], 0x130, 0xf, 0xf, false);
        const bool desc = (inn[u][0] && nx0 < v[u][0]) || (inn[u][1] && nx1 < v[u][1]);
        int mn, mx;
        if (__ballot(desc) == 0) {
          // non-decreasing line: first and last ID (last at offset nin - 1)
          const int nin = __popcll(__ballot(in[u][0])) + __popcll(__ballot(in[u][1]));
          const int last = nin > 0 ? nin - 1 : 0;
          mn = __builtin_amdgcn_readlane(v[u][0], 0);
          mx = last < 64 ? __builtin_amdgcn_readlane(v[u][0], last) : __builtin_amdgcn_readlane(v[u][1], last - 64);
        } else {
          any_desc = true;
          mn = 0x7fffffff;
          mx = (int)0x80000000;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (in[u][h]) {
              mn = min(mn, v[u][h]);
              mx = max(mx, v[u][h]);
            }
          mn = __ockl_wfred_min_i32(mn);
          mx = __ockl_wfred_max_i32(mx);
        }
        if (lane == 0 && l0 + u < nl) {
          stat_s[2 * (l0 + u)] = mn;
          stat_s[2 * (l0 + u) + 1] = mx;
        }
      }
      if (any_desc && lane == 0) *unsorted_s = 1;
    }
  }
  __syncthreads();

  // order across lines: each line's IDs must not be below the previous line's on the same
  // side, and when the query positions start at or after the last key the query side
  // must not be below the key side (otherwise the two ranges overlap and each being
  // ordered orders their union)
  {
    for (int line = tid; line < nl; line += 1024) {
      const bool qside = line < nq;
      const int idx = qside ? line : line - nq;
      const int per = qside ? p.nqb : p.nkb;
      const int blk = idx % per;
      bool bad = blk > 0 && stat_s[2 * line] < stat_s[2 * (line - 1) + 1];
      if (qside && blk == 0 && p.q_offset >= p.kv_len) {
        const int tb = idx / per;
        bad = bad || stat_s[2 * line] < stat_s[2 * (nq + tb * p.nkb + p.nkb - 1) + 1];
      }
      if (bad) *unsorted_s = 1;
    }
  }
}

// Phase 1, sorted IDs: whether the document IDs are non-decreasing over every position
// either side reads (*unsorted_s = 1 when not: a descent inside the query positions or
// inside the key positions of a table group, or, when the query positions start at or
// after the last key, a query ID below the last key's), and each block line's first and
// last ID, which are its minimum and maximum when they are.  Every thread tests eight
// neighbour pairs per side and pass, all loads of a pass issued before any test.
__device__ void doc_ends(const BuildParams& p, int32_t* stat_s, int32_t* unsorted_s) {
  const int tid = threadIdx.x;
  const int nq = p.tB * p.nqb, nl = nq + p.tB * p.nkb;
  constexpr int U = 8;
  bool bad = false;
  for (int tb = 0; tb < p.tB; ++tb) {
    const int32_t* d = doc_row(p.doc, tb);
    const int64_t nqp = p.q_len - 1, nkp = p.kv_len - 1;   // neighbour pairs per side
    for (int64_t base = 0; base < max(nqp, nkp); base += 1024 * U) {
      // loads at clamped positions (a side without pairs reads nothing), so that all of
      // them are in flight at once
      int a[2][U] = {}, b[2][U] = {};
      bool in[2][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t x = base + tid + 1024 * u;
        in[0][u] = x < nqp;
        in[1][u] = x < nkp;
      }
      if (nqp > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t xq = p.q_offset + min(base + tid + 1024 * u, nqp - 1);
          a[0][u] = d[xq];
          b[0][u] = d[xq + 1];
        }
      }
      if (nkp > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t xk = min(base + tid + 1024 * u, nkp - 1);
          a[1][u] = d[xk];
          b[1][u] = d[xk + 1];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) bad = bad || (in[0][u] && b[0][u] < a[0][u]) || (in[1][u] && b[1][u] < a[1][u]);
    }
    if (tid == 0 && p.q_offset >= p.kv_len && p.q_len > 0 && p.kv_len > 0 && d[p.q_offset] < d[p.kv_len - 1])
      bad = true;
  }
  if (bad) *unsorted_s = 1;
  // first and last ID of every line
  for (int line = tid; line < nl; line += 1024) {
    const bool qside = line < nq;
    const int idx = qside ? line : line - nq;
    const int per = qside ? p.nqb : p.nkb;
    const int tb = p.tB == 1 ? 0 : idx / per, blk = idx - tb * per;
    const int32_t* d = doc_row(p.doc, tb);
    int64_t lo, hi;
    if (qside) {
      lo = (int64_t)blk * p.bq + p.q_offset;
      hi = min((int64_t)(blk + 1) * p.bq, p.q_len) + p.q_offset;
    } else {
      lo = (int64_t)blk * p.bk;
      hi = min((int64_t)(blk + 1) * p.bk, p.kv_len);
    }
    stat_s[2 * line] = d[lo];
    stat_s[2 * line + 1] = d[hi - 1];
  }
}

__global__ __launch_bounds__(1024) void build_small_kernel(BuildParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t grid_s[kSmallMaxBlocks];
  __shared__ int32_t stat_s[2 * kSmallMaxLines];   // doc min/max: query blocks, then KV blocks
  __shared__ int32_t cnt_s[2 * kSmallMaxLines];    // partial/full counts: rows, then columns
  __shared__ int32_t pre_s[2 * kSmallMaxLines];    // exclusive prefix of cnt_s within each tb
  __shared__ int32_t tot_s[4 * kSmallMaxTB];       // per tb: rows partial/full, cols partial/full
  __shared__ int32_t cum_s[4 * (kSmallMaxTB + 1)]; // prefix over tb of tH * tot_s
  __shared__ int32_t list_s[kSmallMaxBlocks];      // undecided block ids
  __shared__ int32_t n_undecided;
  __shared__ int32_t unsorted_s;   // some document ID decreases along the positions read
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
  const int nq = p.tB * p.nqb, nl = nq + p.tB * p.nkb;
  const int total = p.tB * p.nqb * p.nkb;
  // every block starts EMPTY and every count at zero
  for (int x = tid; x < (total + 3) / 4; x += 1024) reinterpret_cast<uint32_t*>(grid_s)[x] = 0u;
  for (int x = tid; x < 2 * nl; x += 1024) cnt_s[x] = 0;
  if (tid == 0) {
    unsorted_s = 0;
    n_undecided = 0;
  }
  __syncthreads();

  // phase 1: document-ID ranges per block line, from the lines' end IDs when the IDs are
  // sorted, else by reduction over every ID
  if (p.prog.has_doc) {
    doc_ends(p, stat_s, &unsorted_s);
    __syncthreads();
    if (uniform(unsorted_s) != 0) doc_ranges(p, stat_s, &unsorted_s);
    __syncthreads();
  }
  const bool docs_sorted = p.prog.has_doc && uniform(unsorted_s) == 0;

  // phase 2: one wave per row (tb, r).  For and-only programs the row's possible columns
  // form one band: the allowed keys of a row i are [lo(i), hi(i)], both ends
  // non-decreasing and consecutive rows' intervals touching, so the union over the
  // block's rows a..bb is [lo(a), hi(bb)] and every block outside it is EMPTY.  Blocks
  // in the band (all blocks for programs with an or-node) are classified from their
  // bounds, one per lane; the row's counts come from ballots, the columns' from LDS
  // atomics, and undecided blocks go to a list (its order is irrelevant: each entry's
  // class is decided on its own).
  // positions below 2^30 take 32-bit arithmetic with the row's quantities hoisted
  const bool pos32 = p.prog.mk != MK_GENERIC && p.q_offset + p.q_len < (1ll << 30) && p.kv_len < (1ll << 30);
  const int bk_sh = __builtin_ctz(p.bk);   // block sizes are powers of two
  for (int row = wv; row < nq; row += 16) {
    const int tb = p.tB == 1 ? 0 : row / p.nqb, r = row - tb * p.nqb;
    int c_lo = 0, c_hi = p.nkb - 1;
    const BlockGeom g = geom(p, r, 0);
    if (p.prog.mk != MK_GENERIC) {
      const int64_t lo = p.prog.wmin > 0 ? max((int64_t)0, g.a - p.prog.wmin + 1) : (int64_t)0;
      c_lo = (int)min(lo >> bk_sh, (int64_t)p.nkb);
      if (p.prog.hi_self || p.prog.pmin >= 0) {
        const int64_t hi = p.prog.hi_self ? g.bb : max((int64_t)p.prog.pmin - 1, g.bb);
        c_hi = (int)min(hi >> bk_sh, (int64_t)p.nkb - 1);
      }
    }
    // row quantities of the 32-bit form: lo(bb) and hi(a) (hi unbounded: INT_MAX)
    const int a32 = (int)g.a, bb32 = (int)g.bb;
    const int lo_bb = p.prog.wmin > 0 ? max(0, bb32 - p.prog.wmin + 1) : 0;
    const int hi_a = p.prog.hi_self ? a32 : (p.prog.pmin >= 0 ? max(p.prog.pmin - 1, a32) : 0x7fffffff);
    int np = 0, nf = 0;
    for (int c0 = c_lo; c0 <= c_hi; c0 += 64) {
      const int c = c0 + lane;
      const bool in = c <= c_hi;
      int v = VF;
      if (in) {
        const int32_t* qs = stat_s + 2 * row;
        const int32_t* ks = stat_s + 2 * (nq + tb * p.nkb + c);
        if (pos32) {
          const int k0 = c * p.bk, k1 = min(k0 + p.bk, (int)p.kv_len) - 1;
          v = classify_interval32(p.prog, a32, bb32, lo_bb, hi_a, k0, k1, qs, ks, docs_sorted);
        } else {
          v = classify_bounds(p, geom(p, r, c), qs, ks, docs_sorted);
        }
        if (v == VT || v == VM) {
          grid_s[row * p.nkb + c] = v == VT ? kFull : kPartial;
          atomicAdd(&cnt_s[2 * (nq + tb * p.nkb + c) + (v == VT ? 1 : 0)], 1);
        } else if (v == VU) {
          list_s[atomicAdd(&n_undecided, 1)] = (row << 16) | c;
        }
      }
      np += __popcll(__ballot(v == VM));
      nf += __popcll(__ballot(v == VT));
    }
    if (lane == 0) {
      cnt_s[2 * row] = np;
      cnt_s[2 * row + 1] = nf;
    }
  }
  __syncthreads();

  // phase 3: exact evaluation of the undecided blocks, spread over the 16 waves; the
  // document IDs of a wave's next block are loaded while the current one is decided
  const int nu = uniform(n_undecided);
  // entries are (row << 16) | column (rows below kSmallMaxLines, columns below 2^16)
  auto decode_id = [&](int uid, int& tb, int& r, int& c) {
    const int row = uid >> 16;
    tb = p.tB == 1 ? 0 : row / p.nqb;
    r = row - tb * p.nqb;
    c = uid & 0xffff;
  };
  if (wv < nu) {
    int tb, r, c;
    decode_id(uniform(list_s[wv]), tb, r, c);
    BlockDocs cur = load_block_docs(p, tb, r, c, lane);
    for (int k = wv; k < nu; k += 16) {
      const int uid = uniform(list_s[k]);
      decode_id(uid, tb, r, c);
      BlockDocs nxt = {0, 0, 0, 0};
      if (k + 16 < nu) {
        int tb2, r2, c2;
        decode_id(uniform(list_s[k + 16]), tb2, r2, c2);
        nxt = load_block_docs(p, tb2, r2, c2, lane);
      }
      const uint8_t cls = exact_block(p, tb, r, c, lane, cur);
      if (lane == 0 && cls != kEmpty) {
        grid_s[(tb * p.nqb + r) * p.nkb + c] = cls;
        const int kind = cls == kFull ? 1 : 0;
        atomicAdd(&cnt_s[2 * (tb * p.nqb + r) + kind], 1);
        atomicAdd(&cnt_s[2 * (nq + tb * p.nkb + c) + kind], 1);
      }
      cur = nxt;
    }
  }
  __syncthreads();

  compact_small(p, grid_s, cnt_s, pre_s, tot_s, cum_s, true);
}

// ---------------------------------------------------------------------------------
// Row slices of prebuilt tables: decode takes the query block of the current position
// out of tables built once for the longest context ("FlexAttention: from rules to fused
// kernels", section 5.2), and a shorter square crop is the top-left corner of the longer
// one (same page, section 2.2).  New block (k, c) covers the same or fewer pairs than
// prebuilt block (r_base + k, c), so an EMPTY block stays empty and a FULL one stays
// full, and where the two blocks cover the same pairs a PARTIAL block stays partial.
// Only PARTIAL blocks whose row or key range changed (the ragged last row or column,
// or rows inside a prebuilt block) are decided again, by the builder's own bounds and
// exact evaluation on the new geometry; the rule is evaluated nowhere else.  The result
// equals the tables built for the new geometry.
// ---------------------------------------------------------------------------------
constexpr int kSliceMaxLines = 4096;   // tables B*H * (NQB + NKB)
constexpr int kSliceMaxTB = 256;       // tables B*H

__device__ __forceinline__ bool cell_changes(const SliceParams& sp, int k, int c) {
  const BuildParams& p = sp.d;
  const int64_t r = (int64_t)sp.r_base + k;
  const int64_t a_new = p.q_offset + (int64_t)k * p.bq;
  const int64_t e_new = p.q_offset + min((int64_t)(k + 1) * p.bq, p.q_len);
  const int64_t a_old = sp.src_q_offset + r * p.bq;
  const int64_t e_old = sp.src_q_offset + min((r + 1) * p.bq, sp.src_q_len);
  const int64_t ce = ((int64_t)c + 1) * p.bk;
  return a_new != a_old || e_new != e_old || min(ce, p.kv_len) != min(ce, sp.src_kv_len);
}

// One wave: the classes of new row `row` into g[0, nkb) (cleared beforehand).  Source
// lists are ascending, so each ends at its first column past the new key range.
__device__ void mark_row(const SliceParams& sp, int row, int lane, uint8_t* g) {
  const BuildParams& p = sp.d;
  const int bh = row / p.nqb, k = row - bh * p.nqb;
  const int sl = bh * sp.nqb_src + sp.r_base + k;
  const int b_doc = bh / sp.H;
  {
    const int n = sp.s_num[1][sl];
    const int32_t* a = sp.s_idx[1] + sp.s_ptr[1][sl];
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < n ? a[e] : 0x7fffffff;
      if (c < p.nkb) g[c] = kFull;
      if (__ballot(c < p.nkb) != ~0ull) break;
    }
  }
  const int n = sp.s_num[0][sl];
  const int32_t* a = sp.s_idx[0] + sp.s_ptr[0][sl];
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane;
    const int c = e < n ? a[e] : 0x7fffffff;
    const bool in = c < p.nkb;
    uint8_t cls = kPartial;
    bool need = in && cell_changes(sp, k, c);
    if (need && !p.prog.has_doc) {
      const int v = classify_bounds(p, geom(p, k, c), nullptr, nullptr);
      if (v != VU) {
        cls = v == VT ? kFull : (v == VF ? kEmpty : kPartial);
        need = false;
      }
    }
    // the rest (document rules, undecided or-combinations): the whole wave per block
    uint64_t m = __ballot(need);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const int cc = __builtin_amdgcn_readlane(c, l);
      const uint8_t x = exact_block(p, b_doc, k, cc, lane, load_block_docs(p, b_doc, k, cc, lane));
      if (lane == l) cls = x;
    }
    if (in && cls != kEmpty) g[c] = cls;
    if (__ballot(in) != ~0ull) break;
  }
}

// Tables from selector output ("FlexAttention: from rules to fused kernels", sections
// 5.2 and 6.3): the candidates of a row are range-checked, and each in-range candidate
// block is classified under the rule (bounds, then the exact wavefront walk) and marked
// into the class grid, which sorts the row and makes repeats collapse.
__device__ void mark_row(const SelectParams& sp, int row, int lane, uint8_t* g) {
  const BuildParams& p = sp.d;
  const int bh = row / p.nqb, r = row - bh * p.nqb;
  const int b_doc = bh / sp.H;
  const int32_t* cand = sp.sel + (int64_t)row * sp.k;
  for (int e0 = 0; e0 < sp.k; e0 += 64) {
    const int e = e0 + lane;
    const int c = e < sp.k ? cand[e] : -1;
    const bool in = c >= 0 && c < p.nkb;
    uint8_t cls = kEmpty;
    bool need = in;
    if (in && !p.prog.has_doc) {
      const int v = classify_bounds(p, geom(p, r, c), nullptr, nullptr);
      if (v != VU) {
        cls = v == VT ? kFull : (v == VF ? kEmpty : kPartial);
        need = false;
      }
    }
    uint64_t m = __ballot(need);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const int cc = __builtin_amdgcn_readlane(c, l);
      const uint8_t x = exact_block(p, b_doc, r, cc, lane, load_block_docs(p, b_doc, r, cc, lane));
      if (lane == l) cls = x;
    }
    if (in && cls != kEmpty) g[c] = cls;   // repeats write the same class
  }
}

// One workgroup: the rows are marked into an LDS class grid, then compacted by the
// builder's own counting, prefix and scatter phases.
template <class MP>
__global__ __launch_bounds__(1024) void marked_small_kernel(MP sp) {
  __shared__ __attribute__((aligned(16))) uint8_t grid_s[kSmallMaxBlocks];
  __shared__ int32_t cnt_s[2 * kSliceMaxLines];
  __shared__ int32_t pre_s[2 * kSliceMaxLines];
  __shared__ int32_t tot_s[4 * kSliceMaxTB];
  __shared__ int32_t cum_s[4 * (kSliceMaxTB + 1)];
  const BuildParams& p = sp.d;
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
  const int total = p.tB * p.nqb * p.nkb;
  for (int x = tid; x < (total + 3) / 4; x += 1024) reinterpret_cast<uint32_t*>(grid_s)[x] = 0u;
  __syncthreads();
  for (int row = wv; row < p.tB * p.nqb; row += 16) mark_row(sp, row, lane, grid_s + row * p.nkb);
  __syncthreads();
  compact_small(p, grid_s, cnt_s, pre_s, tot_s, cum_s, false);
}

// larger grids: the class grid goes to the workspace (cleared here, then marked one
// wave per row) and the builder's count, scan and scatter launches compact it
__global__ __launch_bounds__(256) void grid_clear_kernel(uint4* grid, int64_t n16) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n16) grid[t] = make_uint4(0u, 0u, 0u, 0u);
}

template <class MP>
__global__ __launch_bounds__(256) void marked_rows_kernel(MP sp) {
  const BuildParams& p = sp.d;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.tB * p.nqb) return;
  mark_row(sp, row, threadIdx.x & 63, p.grid + (int64_t)row * p.nkb);
}

// Work order: workgroup (tb, x) ranks rows 16 x .. 16 x + 15 of table group tb (rows
// (tb, h, r) for its tH heads, which hold the same rows), one per wave, by descending
// executed-block count, ties by descending index.
__global__ __launch_bounds__(1024) void order_kernel(BuildParams p) {
  __shared__ int32_t len_s[kOrderMaxRows];
  const int tb = blockIdx.x;
  const int64_t base = (int64_t)tb * p.tH * p.nqb;
  for (int r = threadIdx.x; r < p.nqb; r += 1024) len_s[r] = p.kv_num[base + r] + p.full_kv_num[base + r];
  __syncthreads();
  const int r = (int)blockIdx.y * 16 + uniform(threadIdx.x >> 6);
  if (r < p.nqb) rank_row(p, tb, r, threadIdx.x & 63, [&](int y) { return len_s[y]; });
}

inline unsigned waves_to_blocks(int64_t waves) { return (unsigned)((waves + 3) / 4); }

hipError_t launch_order(const BuildParams& p, hipStream_t s) {
  if (p.order && p.tB > 0 && p.nqb > 0)
    hipLaunchKernelGGL(order_kernel, dim3(p.tB, (p.nqb + 15) / 16), dim3(1024), 0, s, p);
  return hipGetLastError();
}

// the one-workgroup writers rank short groups themselves (compact_small)
hipError_t launch_order_after_small(const BuildParams& p, hipStream_t s) {
  return p.nqb <= kOrderInlineRows ? hipGetLastError() : launch_order(p, s);
}


}  // namespace

size_t build_workspace_bytes(int64_t tB, int64_t nqb, int64_t nkb) {
  const size_t grid = (size_t)(tB * nqb * nkb + 255) & ~(size_t)255;
  const size_t stats = (size_t)tB * (nqb + nkb) * 2 * sizeof(int32_t);
  return grid + ((stats + 255) & ~(size_t)255);
}

hipError_t launch_build(const BuildParams& p, hipStream_t s) {
  // an empty grid still gets its counts and pointers (all zero) written
  const int64_t total = (int64_t)p.tB * p.nqb * p.nkb;
  const int64_t lines = (int64_t)p.tB * (p.nqb + p.nkb);
  const int64_t expanded = (int64_t)p.tB * p.tH * (p.nqb + p.nkb);
  if (total <= kSmallMaxBlocks && lines <= kSmallMaxLines && p.tB <= kSmallMaxTB && expanded <= (1 << 20)) {
    hipLaunchKernelGGL(build_small_kernel, dim3(1), dim3(1024), 0, s, p);
    return launch_order_after_small(p, s);
  }
  if (lines > 0 && p.prog.has_doc)
    hipLaunchKernelGGL(doc_stats_kernel, dim3(waves_to_blocks(lines)), dim3(256), 0, s, p);
  if (total > 0)
    hipLaunchKernelGGL(classify_kernel, dim3(waves_to_blocks((total + kClassifyPerWave - 1) / kClassifyPerWave)), dim3(256), 0, s, p);
  if (lines > 0) hipLaunchKernelGGL(count_kernel, dim3(waves_to_blocks(lines)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(scan_kernel, dim3(4), dim3(1024), 0, s, p);
  if (expanded > 0) hipLaunchKernelGGL(scatter_kernel, dim3(waves_to_blocks(expanded)), dim3(256), 0, s, p);
  return launch_order(p, s);
}

size_t slice_workspace_bytes(int64_t tBH, int64_t nqb, int64_t nkb) {
  return (size_t)(tBH * nqb * nkb + 255) & ~(size_t)255;
}

namespace {

template <class MP>
hipError_t launch_marked(const MP& sp, hipStream_t s) {
  const BuildParams& p = sp.d;
  const int64_t total = (int64_t)p.tB * p.nqb * p.nkb;
  const int64_t lines = (int64_t)p.tB * (p.nqb + p.nkb);
  if (total <= kSmallMaxBlocks && lines <= kSliceMaxLines && p.tB <= kSliceMaxTB) {
    hipLaunchKernelGGL(marked_small_kernel<MP>, dim3(1), dim3(1024), 0, s, sp);
    return launch_order_after_small(p, s);
  }
  const int64_t n16 = (total + 15) / 16;   // the workspace is rounded up to 256 bytes
  const int64_t rows = (int64_t)p.tB * p.nqb;
  const int64_t out_lines = rows + (p.q_num ? (int64_t)p.tB * p.nkb : 0);
  if (n16 > 0) {
    hipLaunchKernelGGL(grid_clear_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<uint4*>(p.grid), n16);
    hipLaunchKernelGGL(marked_rows_kernel<MP>, dim3(waves_to_blocks(rows)), dim3(256), 0, s, sp);
  }
  if (out_lines > 0) hipLaunchKernelGGL(count_kernel, dim3(waves_to_blocks(out_lines)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(scan_kernel, dim3(4), dim3(1024), 0, s, p);
  if (out_lines > 0) hipLaunchKernelGGL(scatter_kernel, dim3(waves_to_blocks(out_lines)), dim3(256), 0, s, p);
  return launch_order(p, s);
}

}  // namespace

hipError_t launch_slice(const SliceParams& sp, hipStream_t s) { return launch_marked(sp, s); }

hipError_t launch_select(const SelectParams& sp, hipStream_t s) { return launch_marked(sp, s); }

}  // namespace fa
