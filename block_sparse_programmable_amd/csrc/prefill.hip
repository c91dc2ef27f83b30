// Block-sparse attention forward, prefill shape (many query rows), for gfx950.
//
// One workgroup owns one query block (b, h_q, r) and walks the KV blocks that the
// block table lists for its row: first the FULL list, then the PARTIAL list
// ("FlexAttention: compiler optimization of custom attention", section 3 -- the
// forward fixes a query tile, reads the KV block numbers from the BlockMask and, for
// each kept block, computes Q K^T * scale, applies score_mod, applies mask_mod only
// on partial blocks, then updates the online softmax and accumulates with V).
// Online softmax state and merge law: "Kernels: turning logical sparsity into real
// speed", section 3; "Flash Attention self-test answers", Q24-Q29.  Skipping blocks
// and masking before the row statistics: "FlexAttention: from rules to fused
// kernels", section 3.1.
//
// gfx950 mapping
//   * waves: NW = block_q / 32; wave w owns 32 query rows.  Scores are computed
//     transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so that every lane holds
//     one query row (column) and 16 keys per 32-key tile: row max / row sum stay in
//     the lane apart from one exchange between the two 32-lane halves.
//   * O is accumulated transposed as well (O^T = V^T P^T): P^T in the MFMA output
//     layout feeds the B operand directly once the key order inside each 16-key step
//     is permuted the same way for the V^T operand; the exp work of each 16-key step
//     is interleaved with the P V MFMAs of that step.
//   * K and V are staged in 64-key sub-tiles, both row-major in LDS, copied HBM -> LDS
//     with global_load_lds_dwordx4 (no staging registers, no VALU).  Each lane picks the
//     global 16-byte chunk that its fixed LDS slot must hold, which realises the XOR
//     swizzles: K 16-byte chunks by key & 7 (conflict-free ds_read_b128 fragments), V
//     32-byte units by key & 7 (conflict-free transposing reads).  The P V operand (8
//     keys of one head-dim index per lane) comes from two ds_read_b64_tr_b16 reads.
//     Two LDS slots per operand: sub-tile s+1 is in flight while s is computed, one
//     barrier per sub-tile.
//   * softmax runs in base 2.  Where score_mod is monotone in the raw score (identity,
//     soft-cap, a saturated relative-position bias) the row maximum is taken on the raw
//     MFMA output and mapped once per row; the scale folds into the FMA feeding exp2.
//   * the running maximum is refreshed only when a row's tile maximum exceeds it by
//     more than 2^8 (in base 2), so the O rescale is rare; the normaliser and O use the
//     same reference, which keeps the result exact while bounding every weight by 2^8.
//   * partial blocks: the mask rule is pre-compiled on the host into a per-row key
//     interval (intersections of causal / window / prefix) plus an optional document
//     compare against IDs staged in LDS; other programs use the generic interpreter.
//   * grid order: longest rows first (query block index descending), and heads
//     grouped so that consecutive workgroups of one XCD share a KV head.
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int KT = 64;                 // keys per sub-tile
constexpr int kRelposLdsMax = 3073;    // table entries staged in LDS (2R+1 <= this)
constexpr float kRescaleThresh = 8.0f; // base-2 growth allowed before rescaling O

template <int D>
struct Lds {
  static constexpr int KROW = D * 2;          // bytes per K or V row
  static constexpr int TILE = KT * KROW;      // one K or one V sub-tile
  static constexpr int UNITS = D / 16;        // 32-byte units per V row
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kListCap = 512;   // block-list entries staged in LDS per pass over the row

// K: physical 16-byte chunk of row `key` holding logical chunk `ch`
__device__ __forceinline__ int k_off(int key, int ch, int krow) { return key * krow + ((ch ^ (key & 7)) << 4); }
// V: byte offset of V[key][d] (d a multiple of 4) with 32-byte units XOR-swizzled by key & 7
template <int D>
__device__ __forceinline__ int v_off(int key, int d) {
  constexpr int UM = Lds<D>::UNITS - 1;
  return key * (D * 2) + ((((d >> 4) ^ (key & 7)) & UM) << 5) + ((d & 15) << 1);
}

// key offset (within the 64-key sub-tile) held by S^T register rr of M-tile mt,
// excluding the lane-half term 4*half
__device__ __forceinline__ constexpr int key_of(int mt, int rr) { return 32 * mt + 8 * (rr >> 2) + (rr & 3); }

template <int... U, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, U...>, F&& f) {
  (f(std::integral_constant<int, U>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// LDS byte address of a __shared__ object (the M0 operand of the LDS-DMA loads)
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const lds_void*)ptr;
}

// HBM -> LDS loads that bypass VGPRs (global_load_lds).  Lane l writes LDS bytes
// [m0 + IMM + 16 l, +16); the immediate offset applies to the global and the LDS side
// alike.  Issued from inline assembly so that every address is a scalar base plus one
// precomputed per-lane offset; the caller waits (vmcnt) before the barrier that
// publishes the tile.  One wait state separates the M0 write from the load that reads
// it.
// wave-uniform value in scalar registers (the "s" operands below)
__device__ __forceinline__ uint32_t sreg(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const void* sreg(const void* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint64_t lo = sreg((uint32_t)v), hi = sreg((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(lo | (hi << 32));
}

template <int IMM>
__device__ __forceinline__ void dma16_s(uint32_t m0, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3"
               :: "s"(sreg(m0)), "v"(voff), "s"(sreg(sbase)), "i"(IMM) : "memory", "m0");
}
__device__ __forceinline__ void dma16_v(uint32_t m0, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(sreg(m0)), "v"(gaddr) : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(uint32_t m0, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(sreg(m0)), "v"(voff), "s"(sreg(sbase)) : "memory", "m0");
}
__device__ __forceinline__ void dma4_v(uint32_t m0, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(sreg(m0)), "v"(gaddr) : "memory", "m0");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// round-to-nearest-even pair conversion into one dword (v_cvt_pk_bf16_f32), low = a
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int D, int NW, int SCORE, int MK>
__global__ __launch_bounds__(NW * 64, 2) void prefill_kernel(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int KSTEPS = D / 16; // k-steps of the QK^T product
  constexpr int DM = D / 32;     // 32-row tiles of O^T
  constexpr int KPK = 1024 / (D * 2);       // keys covered by one 1 KB wave copy
  constexpr int COPIES = KT / KPK / NW;     // 1 KB copies per wave per operand
  constexpr int VAR = KPK >= 8 ? 1 : 8 / KPK;  // distinct swizzle patterns over the copies
  constexpr bool kDoc = (MK == MK_INTERVAL_DOC);
  constexpr bool kRel = (SCORE == FA_S_RELPOS);
  using L = Lds<D>;
  static_assert(L::KROW * KPK == 1024, "one copy moves 1 KB");
  static_assert((COPIES * KPK) % 8 == 0, "wave slices start at a multiple of 8 keys");
  // K slot 0 | K slot 1 | V slot 0 | V slot 1 | doc IDs slot 0 | slot 1.  The loop below is
  // unrolled by two, so every LDS read is a per-lane base plus an immediate offset.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * L::TILE + 2 * KT * 4];
  __shared__ int32_t list_s[kListCap];
  __shared__ float rel_lds[kRel ? kRelposLdsMax : 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (b, h_q, r), longest rows first, heads grouped per XCD
  const int nbh = p.B * p.Hq;
  const int nqb = p.tab.nqb;
  const int Lid = blockIdx.x;
  int bh, r;
  if ((nbh & 7) == 0) {
    const int per = nbh >> 3, x = Lid & 7, jj = Lid >> 3;
    bh = x * per + jj % per;
    r = nqb - 1 - jj / per;
  } else {
    bh = Lid % nbh;
    r = nqb - 1 - Lid / nbh;
  }
  const int b = bh / p.Hq;
  const int hq = bh - b * p.Hq;
  const int hkv = hq / p.g;

  const int q_len = (int)p.q_len;
  const int kv_len = (int)p.kv_len;
  const int i_loc = r * BQ + w * 32 + col;
  const bool row_ok = i_loc < q_len;
  const int i_g = i_loc + (int)p.q_offset;
  const int i_wave0 = r * BQ + w * 32 + (int)p.q_offset;   // first row of the wave

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[row][16t + 8 half .. +8]
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + ((int64_t)bh * p.q_len + (row_ok ? i_loc : 0)) * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 v = row_ok ? load16(qrow + 16 * t + 8 * half) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
    // consume the loads here: the block loop's HBM -> LDS copies are invisible to the
    // compiler's wait counting, which would otherwise wait for all memory at every tile
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) asm volatile("" : "+v"(qf[t]));
  }

  // ---- block-table row
  const int tb = p.tab.tB == 1 ? 0 : b;
  const int th = p.tab.tH == 1 ? 0 : hq;
  const int row = (tb * p.tab.tH + th) * nqb + r;
  const int nf = uniform(p.tab.fnum[row]);
  const int np = uniform(p.tab.num[row]);
  const int32_t* flist = p.tab.fidx + uniform(p.tab.fptr[row]);
  const int32_t* plist = p.tab.idx + uniform(p.tab.ptr[row]);
  const int bk = p.tab.bk;
  const int spb_sh = bk == 2 * KT ? 1 : 0;   // sub-tiles per block = 1 << spb_sh
  const int n_ent = nf + np;

  const uint16_t* kbase = p.k + (int64_t)(b * p.Hkv + hkv) * p.kv_len * D;
  const uint16_t* vbase = p.v + (int64_t)(b * p.Hkv + hkv) * p.kv_len * D;
  const int32_t* docr = doc_row(p.doc, b);
  const int doc_i = (p.prog.has_doc && row_ok) ? docr[i_g] : 0;
  const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);

  // per-row allowed key interval of the pre-compiled mask (partial blocks only)
  uint32_t lo_u = 0, span = 0;
  if constexpr (MK != MK_GENERIC) {
    int lo = p.prog.wmin > 0 ? max(0, i_g - p.prog.wmin + 1) : 0;
    int hi = p.prog.hi_self ? i_g : (p.prog.pmin >= 0 ? max(p.prog.pmin - 1, i_g) : 0x7fffffff);
    hi = min(hi, kv_len - 1);
    if (hi >= lo) {
      lo_u = (uint32_t)lo;
      span = (uint32_t)(hi - lo);
    } else {
      lo_u = 0x80000000u;  // no key of any sub-tile can match
      span = 0;
    }
  }

  // relative-position table of this query head, pre-multiplied by log2(e); the two
  // saturated entries are kept in registers
  const int R = p.score.radius;
  const bool rel_in_lds = kRel && (2 * R + 1) <= kRelposLdsMax;
  float bias_far2 = 0.f, bias_ahead2 = 0.f;   // rel >= R and rel <= -R
  if constexpr (kRel) {
    if (rel_in_lds) {
      for (int x = tid; x < 2 * R + 1; x += NT) rel_lds[x] = sc.tab[x] * kLog2e;
    }
    bias_far2 = sc.tab[2 * R] * kLog2e;
    bias_ahead2 = sc.tab[0] * kLog2e;
  }

  // ---- per-lane offsets of the HBM -> LDS copies.  Wave w fills keys
  // [w COPIES KPK, (w+1) COPIES KPK) of a sub-tile, 1 KB (KPK keys) per copy; LDS slots are
  // linear, and each lane fetches the global chunk its slot must hold under the swizzle.
  const int wu = uniform(w);
  const int wave_key0 = wu * COPIES * KPK;
  uint32_t koff[VAR], voff[VAR];
#pragma unroll
  for (int var = 0; var < VAR; ++var) {
    const int key_in = lane / DCH;
    const int pc = lane % DCH;
    const int key7 = (var * KPK + key_in) & 7;
    koff[var] = (uint32_t)(key_in * L::KROW + ((pc ^ key7) << 4));
    voff[var] = (uint32_t)(key_in * L::KROW + ((2 * (((pc >> 1) ^ key7) & (L::UNITS - 1)) + (pc & 1)) << 4));
  }

  auto copy_tile = [&](int j0, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    const uint32_t mk = lds_addr(smem + SLOT * L::TILE) + wave_key0 * L::KROW;
    const uint32_t mv = lds_addr(smem + (2 + SLOT) * L::TILE) + wave_key0 * L::KROW;
    const uint32_t md = lds_addr(smem + 4 * L::TILE + SLOT * KT * 4);
    if (j0 + KT <= kv_len) {
      const char* kg = (const char*)kbase + ((int64_t)j0 + wave_key0) * L::KROW;
      const char* vg = (const char*)vbase + ((int64_t)j0 + wave_key0) * L::KROW;
      static_for<COPIES>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int grp = (u / 4) * 4096;   // immediate offsets stay below 4 KB
        dma16_s<(u % 4) * 1024>(mk + grp, kg + grp, koff[u % VAR]);
        dma16_s<(u % 4) * 1024>(mv + grp, vg + grp, voff[u % VAR]);
      });
      if constexpr (kDoc) {
        if (wu == 0) dma4_s(md, docr + j0, (uint32_t)lane * 4);
      }
    } else {
      // ragged tail: keys past kv_len re-read the last key (they are masked)
      static_for<COPIES>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int key = wave_key0 + u * KPK + lane / DCH;
        const int64_t j = min(j0 + key, kv_len - 1);
        dma16_v(mk + u * 1024, (const char*)kbase + j * L::KROW + (koff[u % VAR] & (L::KROW - 1)));
        dma16_v(mv + u * 1024, (const char*)vbase + j * L::KROW + (voff[u % VAR] & (L::KROW - 1)));
      });
      if constexpr (kDoc) {
        if (wu == 0) dma4_v(md, docr + min(j0 + lane, kv_len - 1));
      }
    }
  };

  // ---- per-lane LDS read bases.  K fragment (mt, t): key 32 mt + col, logical chunk
  // 2t + half at physical chunk (2t + half) ^ (key & 7); t = 4q + t' adds q * 128 bytes.
  // V^T fragment (t, dm, hl): keys 16 t + 8 hl + 4 half + (li >> 2), head-dim d0 =
  // 32 dm + 16 (g16 & 1) + 4 (li & 3); t and hl add whole rows.
  const int g16 = lane >> 4, li = lane & 15;
  uint32_t kaddr[4], vaddr[DM];
#pragma unroll
  for (int t = 0; t < 4; ++t) kaddr[t] = (uint32_t)k_off(col, 2 * t + half, L::KROW);
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
    vaddr[dm] = (uint32_t)v_off<D>(4 * half + (li >> 2), 32 * dm + 16 * (g16 & 1) + 4 * (li & 3));

  // ---- online softmax state (per lane: one query row; halves share m)
  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  // ---- one 64-key sub-tile from LDS (buf, vb, dl); MASKED: partial block or ragged tail
  auto compute = [&](auto slot_c, bool masked, bool part, int j0) {
    constexpr int SLOT = decltype(slot_c)::value;
    const uint8_t* kb = smem + SLOT * L::TILE;
    const uint8_t* vb = smem + (2 + SLOT) * L::TILE;
    const int32_t* dl = reinterpret_cast<const int32_t*>(smem + 4 * L::TILE + SLOT * KT * 4);
    // S^T = K Q^T
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kb + kaddr[t & 3] + (t >> 2) * 128 + mt * 32 * L::KROW);
        sacc[mt] = mfma32(__builtin_bit_cast(bf16x8, kv), qf[t], sacc[mt]);
      }
    }
    const int jl = j0 + 4 * half;   // key of element (mt=0, rr=0) in this lane

    // element mask: x = -inf where disallowed
    if (masked) {
      if constexpr (MK == MK_GENERIC) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int j = jl + key_of(mt, rr);
            bool ok = (unsigned)j < (unsigned)kv_len;
            if (part && ok) ok = mask_allowed(p.prog, i_g, j, doc_i, p.prog.has_doc ? docr[j] : 0);
            sacc[mt][rr] = ok ? sacc[mt][rr] : kNegInf;
          }
      } else {
        // keys outside [lo, hi] (hi already clipped to kv_len - 1) are masked; when only
        // the ragged tail needs masking the same test applies with the tail bound alone
        uint32_t lo_t = lo_u, span_t = span;
        if (!part) {
          lo_t = 0;
          span_t = (uint32_t)(kv_len - 1);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            int dq[4] = {doc_i, doc_i, doc_i, doc_i};
            if constexpr (kDoc) {
              if (part) {
                const u32x4 dv = *reinterpret_cast<const u32x4*>(dl + 32 * mt + 8 * g4 + 4 * half);
                dq[0] = (int)dv[0];
                dq[1] = (int)dv[1];
                dq[2] = (int)dv[2];
                dq[3] = (int)dv[3];
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rr = 4 * g4 + e;
              const uint32_t j = (uint32_t)(jl + key_of(mt, rr));
              const bool ok = (j - lo_t) <= span_t && dq[e] == doc_i;
              sacc[mt][rr] = ok ? sacc[mt][rr] : kNegInf;
            }
          }
      }
    }

    // score_mod to the base-2 domain and the tile maximum.  Monotone kinds keep the raw
    // score in sacc (tile maximum mapped once); the others store
    // t = log2(e) * score_mod(s * scale) in sacc.
    bool raw_mode;
    float bias2 = 0.f;  // constant base-2 bias of a saturated relative-position tile
    if constexpr (SCORE == FA_S_IDENTITY || SCORE == FA_S_SOFTCAP) {
      raw_mode = true;
    } else if constexpr (SCORE == FA_S_RELPOS) {
      const int dmin = i_wave0 - (j0 + KT - 1);
      const int dmax = i_wave0 + 31 - j0;
      raw_mode = dmin >= R || dmax <= -R;
      bias2 = dmin >= R ? bias_far2 : bias_ahead2;
    } else {
      raw_mode = false;
    }
    float tmax = kNegInf;
    if (raw_mode) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, sacc[mt][rr]);
    } else {
      if constexpr (SCORE == FA_S_ALIBI) {
        const float base = sc.slope2 * (float)(jl - i_g);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float t = __builtin_fmaf(sacc[mt][rr], sc.c2, __builtin_fmaf(sc.slope2, (float)key_of(mt, rr), base));
            sacc[mt][rr] = t;
            tmax = fmaxf(tmax, t);
          }
      } else if constexpr (SCORE == FA_S_RELPOS) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            int rel = i_g - (jl + key_of(mt, rr));
            rel = rel < -R ? -R : (rel > R ? R : rel);
            const float bb = rel_in_lds ? rel_lds[rel + R] : sc.tab[rel + R] * kLog2e;
            const float t = __builtin_fmaf(sacc[mt][rr], sc.c2, bb);
            sacc[mt][rr] = t;
            tmax = fmaxf(tmax, t);
          }
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // map a raw-score maximum into the base-2 domain
    float m_cand = tmax;
    if (raw_mode && tmax != kNegInf) {
      if constexpr (SCORE == FA_S_SOFTCAP) {
        m_cand = sc.cap2 - 2.f * sc.cap2 * fast_rcp(fast_exp2(tmax * sc.capk) + 1.f);
      } else {
        m_cand = __builtin_fmaf(tmax, sc.c2, bias2);
      }
    }

    // lazy online-softmax rescale (wave-uniform branch)
    const bool grow = m_cand > m_run + kRescaleThresh;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? m_cand : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;   // 0 when m_run = -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    const float softcap_c = sc.cap2 - m_use;
    const float raw_c = bias2 - m_use;

    // weights P (bf16), row sum and O^T += V^T P^T, one 16-key step at a time
    float psum = 0.f;
    // P for the 8 elements of 16-key step t (packed bf16 pairs); CHECK re-applies the
    // mask where the soft-cap would map a -inf score to a finite value
    auto p_step = [&](int t, u32x4& pk, auto check_c) {
      constexpr bool CHECK = decltype(check_c)::value;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float pv[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float x = sacc[t >> 1][8 * (t & 1) + 2 * e2 + h2];
          float arg;
          if constexpr (SCORE == FA_S_SOFTCAP) {
            const float rr = fast_rcp(fast_exp2(x * sc.capk) + 1.f);
            arg = __builtin_fmaf(-2.f * sc.cap2, rr, softcap_c);
            if constexpr (CHECK) arg = (x == kNegInf) ? kNegInf : arg;
          } else if constexpr (SCORE == FA_S_IDENTITY) {
            arg = __builtin_fmaf(x, sc.c2, -m_use);
          } else {
            arg = raw_mode ? __builtin_fmaf(x, sc.c2, raw_c) : x - m_use;
          }
          pv[h2] = fast_exp2(arg);
        }
        pk[e2] = cvt_pk_bf16(pv[0], pv[1]);
        psum += pv[0] + pv[1];
      }
    };
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pk;
      if (SCORE == FA_S_SOFTCAP && masked) {
        p_step(t, pk, std::true_type{});
      } else {
        p_step(t, pk, std::false_type{});
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
      // V^T fragment rows d = 32 dm + (lane & 31), keys of this step in the slot order
      // of P^T: two transposing reads of 4 keys x 16 head-dim indices per 16-lane group
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const uint8_t* va = vb + vaddr[dm] + 16 * t * L::KROW;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(va + 8 * L::KROW));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dm] = mfma32(a, pb, oacc[dm]);
      }
    }
    l_run += psum;
  };

  // ---- the row's block list (full entries, then partial) in passes of kListCap entries
  for (int c0 = 0; c0 < n_ent; c0 += kListCap) {
    const int cnt = min(kListCap, n_ent - c0);
    for (int e = tid; e < cnt; e += NT) {
      const int ge = c0 + e;
      list_s[e] = ge < nf ? flist[ge] : plist[ge - nf];
    }
    __syncthreads();
    const int nsub = cnt << spb_sh;
    auto sub_j0 = [&](int s, bool& part) -> int {
      const int blk = s >> spb_sh;
      part = c0 + blk >= nf;
      return uniform(list_s[blk]) * bk + (s & spb_sh) * KT;
    };
    bool part_cur = false;
    int j0_cur = sub_j0(0, part_cur);
    copy_tile(j0_cur, std::integral_constant<int, 0>{});
    wait_dma();
    __syncthreads();

    // sub-tile s from one slot while s+1 is copied into the other
    auto step = [&](int s, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      bool part_nxt = false;
      int j0_nxt = 0;
      if (s + 1 < nsub) {
        j0_nxt = sub_j0(s + 1, part_nxt);
        copy_tile(j0_nxt, std::integral_constant<int, 1 - SLOT>{});
      }
      compute(slot_c, part_cur || j0_cur + KT > kv_len, part_cur, j0_cur);
      wait_dma();
      __syncthreads();
      part_cur = part_nxt;
      j0_cur = j0_nxt;
    };
    for (int s = 0; s < nsub; s += 2) {
      step(s, std::integral_constant<int, 0>{});
      if (s + 1 < nsub) step(s + 1, std::integral_constant<int, 1>{});
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    uint16_t* orow = p.o + ((int64_t)bh * p.q_len + i_loc) * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dm + 8 * gq + 4 * half;
        u32x2 o2;
        o2[0] = cvt_pk_bf16(oacc[dm][4 * gq + 0] * inv, oacc[dm][4 * gq + 1] * inv);
        o2[1] = cvt_pk_bf16(oacc[dm][4 * gq + 2] * inv, oacc[dm][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = o2;
      }
    }
    if (half == 0) {
      p.lse[(int64_t)bh * p.q_len + i_loc] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, int NW, int SCORE>
void launch_mk(const FwdParams& p, hipStream_t s, dim3 grid, dim3 block) {
  switch (p.prog.mk) {
    case MK_INTERVAL: hipLaunchKernelGGL((prefill_kernel<D, NW, SCORE, MK_INTERVAL>), grid, block, 0, s, p); break;
    case MK_INTERVAL_DOC: hipLaunchKernelGGL((prefill_kernel<D, NW, SCORE, MK_INTERVAL_DOC>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<D, NW, SCORE, MK_GENERIC>), grid, block, 0, s, p); break;
  }
}

template <int D, int NW>
hipError_t launch_nw(const FwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.Hq * p.tab.nqb));
  const dim3 block(NW * 64);
  switch (p.score.kind) {
    case FA_S_IDENTITY: launch_mk<D, NW, FA_S_IDENTITY>(p, s, grid, block); break;
    case FA_S_ALIBI: launch_mk<D, NW, FA_S_ALIBI>(p, s, grid, block); break;
    case FA_S_SOFTCAP: launch_mk<D, NW, FA_S_SOFTCAP>(p, s, grid, block); break;
    default: launch_mk<D, NW, FA_S_RELPOS>(p, s, grid, block); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdParams& p, hipStream_t s) {
  if (p.B * p.Hq * p.tab.nqb == 0) return hipSuccess;
  const int nw = p.tab.bq / 32;
  if (p.d == 128) return nw == 4 ? launch_nw<128, 4>(p, s) : launch_nw<128, 2>(p, s);
  return nw == 4 ? launch_nw<64, 4>(p, s) : launch_nw<64, 2>(p, s);
}

}  // namespace fa
