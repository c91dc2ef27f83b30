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
//     swizzles of K 16-byte chunks and V 32-byte units, chosen for the 64-bank LDS so
//     that the ds_read_b128 fragments and the transposing reads are free of bank
//     conflicts (an XOR by key & 7 leaves a 2-way conflict).  The P V operand (8
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
//   * grid order: longest rows first -- by the tables' work order when they carry one
//     ("FlexAttention: from rules to fused kernels", section 5.2: bucket query tiles by
//     their executed blocks), else by descending query block index -- and heads grouped
//     so that consecutive workgroups of one XCD share a KV head.
#include "device_common.hpp"
#include "fa_internal.hpp"
#include "prefill_common.hpp"

namespace fa {

namespace {

// soft-cap kernels keep a fixed softmax reference at cap2 = softcap * log2(e) when
// cap2 <= this (softcap <= 34.6): weights then stay within [2^-100, 1]
constexpr float kFixedRefMax = 50.0f;

template <int D, int NW, int SCORE, int MK>
__global__ __launch_bounds__(NW * 64, 2) void prefill_kernel(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int KSTEPS = D / 16; // k-steps of the QK^T product
  constexpr int DM = D / 32;     // 32-row tiles of O^T
  constexpr int KPK = 1024 / (D * 2);       // keys covered by one 1 KB wave copy
  constexpr int COPIES = KT / KPK / NW;     // 1 KB copies per wave per operand
  constexpr int KVAR = KPK >= kSwzKeys ? 1 : kSwzKeys / KPK;  // K swizzle patterns over the copies
  constexpr int VVAR = KPK >= 8 ? 1 : 8 / KPK;                 // V pattern repeats every 8 keys
  constexpr bool kDoc = (MK == MK_INTERVAL_DOC);
  // document IDs of each K sub-tile are staged in LDS next to it when a mask needs them
  // (the generic interpreter only when its program has a document leaf)
  const bool stage_doc = kDoc || (MK == MK_GENERIC && p.prog.has_doc);
  constexpr bool kRel = (SCORE == FA_S_RELPOS);
  using L = Lds<D>;
  static_assert(L::KROW * KPK == 1024, "one copy moves 1 KB");
  static_assert((COPIES * KPK) % kSwzKeys == 0, "wave slices start at a swizzle period");
  // K slot 0 | K slot 1 | V slot 0 | V slot 1 | doc IDs slot 0 | slot 1 (doc IDs travel
  // with K).  Every LDS read is a per-lane base plus an immediate offset.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * L::TILE + 2 * KT * 4];
  __shared__ int32_t list_s[kListCap];
  __shared__ float rel_lds[kRel ? kRelposLdsMax + 2 * kRelPad : 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (b, h_q, r), longest rows first, heads grouped per XCD
  const int nbh = p.B * p.Hq;
  const int nqb = p.tab.nqb;
  const int Lid = blockIdx.x;
  int bh, rank;
  if ((nbh & 7) == 0) {
    const int per = nbh >> 3, x = Lid & 7, jj = Lid >> 3;
    bh = x * per + jj % per;
    rank = jj / per;
  } else {
    bh = Lid % nbh;
    rank = Lid / nbh;
  }
  const int b = bh / p.Hq;
  const int hq = bh - b * p.Hq;
  const int hkv = hq / p.g;
  const int tb = p.tab.tB == 1 ? 0 : b;
  const int th = p.tab.tH == 1 ? 0 : hq;
  // rank-th longest query block of this table entry: from the tables' work order when
  // present, else by descending index (longest first for causal-like rules)
  const int r = p.tab.order ? uniform(p.tab.order[(tb * p.tab.tH + th) * nqb + rank]) : nqb - 1 - rank;

  const int q_len = (int)p.q_len;
  const int kv_len = (int)p.kv_len;
  const int i_loc = r * BQ + w * 32 + col;
  const bool row_ok = i_loc < q_len;
  const int i_g = i_loc + (int)p.q_offset;
  const int i_wave0 = r * BQ + w * 32 + (int)p.q_offset;   // first row of the wave

  // ---- block-table row, read through the constant address space at wave-uniform
  // indexes (scalar loads): it starts the item's longest chain of dependent loads (row
  // -> list entries -> tile copies), so it goes out first
  using cptr = const __attribute__((address_space(4))) int32_t*;
  const int row = (tb * p.tab.tH + th) * nqb + r;
  const int nf = ((cptr)sreg(p.tab.fnum))[row];
  const int np = ((cptr)sreg(p.tab.num))[row];
  const int32_t* flist = p.tab.fidx + ((cptr)sreg(p.tab.fptr))[row];
  const int32_t* plist = p.tab.idx + ((cptr)sreg(p.tab.ptr))[row];
  const int bk = p.tab.bk;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[row][16t + 8 half .. +8].
  // The loads stay in flight until the first tiles have arrived (see the prologue).
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + ((int64_t)bh * p.q_len + (row_ok ? i_loc : 0)) * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 v = row_ok ? load16(qrow + 16 * t + 8 * half) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const int spb_sh = bk == 2 * KT ? 1 : 0;   // sub-tiles per block = 1 << spb_sh
  const int n_ent = nf + np;

  const uint16_t* kbase = p.k + (int64_t)(b * p.Hkv + hkv) * p.kv_len * D;
  const uint16_t* vbase = p.v + (int64_t)(b * p.Hkv + hkv) * p.kv_len * D;
  const int32_t* docr = doc_row(p.doc, b);
  int doc_i = (p.prog.has_doc && row_ok) ? docr[i_g] : 0;
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

  // relative-position table of this query head, entry of offset i - j at index
  // i - j + R + kRelPad, with kRelPad copies of each saturated entry on either side: a
  // tile that is not saturated for the wave spans offsets within 94 of [-R, R], so its
  // reads need no clamping.  The two saturated entries (times log2 e) are also kept in
  // registers.  A table too large for LDS travels as per-tile windows instead: the
  // entries for offsets i - j of the workgroup's rows against a K sub-tile at j0,
  // [wb, wb + BQ + KT - 2] with wb = i_wg0 - j0 - (KT - 1), clamped to [-R, R] at copy
  // time (kRelWin per K slot, copied with the K tile)
  const int R = p.score.radius;
  const bool rel_in_lds = kRel && (2 * R + 1) <= kRelposLdsMax;
  const int i_wg0 = r * BQ + (int)p.q_offset;   // first row of the workgroup
  float bias_far2 = 0.f, bias_ahead2 = 0.f;   // rel >= R and rel <= -R
  if constexpr (kRel) {
    if (rel_in_lds) {
      for (int x = tid; x < 2 * R + 1 + 2 * kRelPad; x += NT)
        rel_lds[x] = sc.tab[min(max(x - kRelPad, 0), 2 * R)];
    }
    bias_far2 = sc.tab[2 * R] * kLog2e;
    bias_ahead2 = sc.tab[0] * kLog2e;
  }

  // ---- per-lane offsets of the HBM -> LDS copies.  Wave w fills keys
  // [w COPIES KPK, (w+1) COPIES KPK) of a sub-tile, 1 KB (KPK keys) per copy; LDS slots are
  // linear, and each lane fetches the global chunk its slot must hold under the swizzle.
  const int wu = uniform(w);
  const int wave_key0 = wu * COPIES * KPK;
  // Both swizzles are XOR-linear in the key and a copy's first key is a multiple of
  // KPK, so the offsets of later copies in a period are the first copy's offsets XOR a
  // constant (flipped next to each copy, which keeps one live register per operand).
  uint32_t koff0, voff0;
  {
    const int key_in = lane / DCH;
    const int pc = lane % DCH;
    koff0 = (uint32_t)(key_in * L::KROW + ((pc ^ k_swz<D>(key_in)) << 4));
    voff0 = (uint32_t)(key_in * L::KROW + ((2 * (((pc >> 1) ^ v_swz<D>(key_in)) & (L::UNITS - 1)) + (pc & 1)) << 4));
  }
  auto copy_off = [&](auto isv_c, auto u_c) -> uint32_t {
    constexpr bool ISV = decltype(isv_c)::value;
    constexpr int u = decltype(u_c)::value;
    constexpr uint32_t flip = ISV ? (uint32_t)(v_swz<D>((u % VVAR) * KPK) << 5)
                                  : (uint32_t)(k_swz<D>((u % KVAR) * KPK) << 4);
    const uint32_t base = ISV ? voff0 : koff0;
    if constexpr (flip == 0) {
      return base;
    } else {
      uint32_t o;
      asm volatile("v_xor_b32 %0, %1, %2" : "=v"(o) : "i"(flip), "v"(base));
      return o;
    }
  };

  // the position-table window of the K sub-tile at j0 (wave 0, three 64-entry copies)
  auto copy_rel_window = [&](int j0, auto isv_c, auto slot_c) {
    if constexpr (kRel && !decltype(isv_c)::value) {
      if (!rel_in_lds && wu == 0) {
        const uint32_t mw = lds_addr(rel_lds + decltype(slot_c)::value * kRelWin);
        const int wb = i_wg0 - j0 - (KT - 1);
#pragma unroll
        for (int u = 0; u < kRelWin / 64; ++u) {
          const int rel = min(max(wb + 64 * u + lane, -R), R);
          dma4_v(mw + 256 * u, sc.tab + rel + R);
        }
      }
    }
  };

  // copy of one operand (K with its doc IDs, or V) of the sub-tile at key j0 into a slot
  auto copy_op = [&](int j0, auto isv_c, auto slot_c) {
    constexpr bool ISV = decltype(isv_c)::value;
    constexpr int SLOT = decltype(slot_c)::value;
    const uint16_t* gb = ISV ? vbase : kbase;
    const uint32_t m = lds_addr(smem + ((ISV ? 2 : 0) + SLOT) * L::TILE) + wave_key0 * L::KROW;
    const uint32_t md = lds_addr(smem + 4 * L::TILE + SLOT * KT * 4);

    if (j0 + KT <= kv_len) {
      const char* g = (const char*)gb + ((int64_t)j0 + wave_key0) * L::KROW;
      static_for<COPIES>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int grp = (u / 4) * 4096;   // immediate offsets stay below 4 KB
        dma16_s<(u % 4) * 1024>(m + grp, g + grp, copy_off(isv_c, uc));
      });
      if constexpr (MK != MK_INTERVAL && !ISV) {
        if (stage_doc && wu == 0) dma4_s(md, docr + j0, (uint32_t)lane * 4);
      }
      copy_rel_window(j0, isv_c, slot_c);
    } else {
      // ragged tail: keys past kv_len re-read the last key (they are masked)
      static_for<COPIES>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int key = wave_key0 + u * KPK + lane / DCH;
        const int64_t j = min(j0 + key, kv_len - 1);
        const uint32_t o = copy_off(isv_c, uc);
        dma16_v(m + u * 1024, (const char*)gb + j * L::KROW + (o & (L::KROW - 1)));
      });
      if constexpr (MK != MK_INTERVAL && !ISV) {
        if (stage_doc && wu == 0) dma4_v(md, docr + min(j0 + lane, kv_len - 1));
      }
      copy_rel_window(j0, isv_c, slot_c);
    }
  };

  // ---- per-lane LDS read bases.  K fragment (mt, t): key 32 mt + col, logical chunk
  // 2t + half at physical chunk (2t + half) ^ k_swz(key); mt adds whole rows.
  // V^T fragment (t, dm, hl): keys 16 t + 8 hl + 4 half + (li >> 2), head-dim d0 =
  // 32 dm + 16 (g16 & 1) + 4 (li & 3); t and hl add whole rows.
  const int g16 = lane >> 4, li = lane & 15;
  // Chunks 8..15 of a 256-byte row sit at the address of chunk - 8 with bit 7 flipped;
  // that XOR is issued next to each read (volatile, so it is not hoisted into 4 more
  // live registers).
  uint32_t kaddr[4], vaddr[DM];
#pragma unroll
  for (int t = 0; t < 4; ++t) kaddr[t] = (uint32_t)k_off<D>(col, 2 * t + half);
  auto kfrag = [&](int t) -> uint32_t {
    if (t < 4) return kaddr[t];
    uint32_t a;
    asm volatile("v_xor_b32 %0, 0x80, %1" : "=v"(a) : "v"(kaddr[t & 3]));
    return a;
  };
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
    vaddr[dm] = (uint32_t)v_off<D>(4 * half + (li >> 2), 32 * dm + 16 * (g16 & 1) + 4 * (li & 3));

  // ---- online softmax state (per lane: one query row; halves share m).  Soft-cap scores
  // never exceed the cap, so with the reference fixed at cap2 every weight lies in
  // [2^(-2 cap2), 1]; for caps with 2 cap2 <= 2 kFixedRefMax that range stays far inside
  // the normal floats and bf16, and the running maximum and its rescales are skipped.
  const bool fixed_ref = SCORE == FA_S_SOFTCAP && sc.cap2 <= kFixedRefMax;
  float m_run = fixed_ref ? sc.cap2 : kNegInf;
  float l_run = 0.f;
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  // ---- accumulator start of the S^T tile at key j0n, M-tile mt: zero, or for ALiBi the
  // bias over the scale, slope (j - i) / scale, so that the product itself carries the
  // bias and the score stays monotone in the accumulator (t = c2 * acc)
  const float alibi_bs = SCORE == FA_S_ALIBI ? sc.slope2 / sc.c2 : 0.f;
  auto acc_start = [&](int j0n, int mt) -> f32x16 {
    f32x16 a = f32x16{};
    if constexpr (SCORE == FA_S_ALIBI) {
      const float base = alibi_bs * (float)(j0n + 4 * half - i_g);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) a[rr] = __builtin_fmaf(alibi_bs, (float)key_of(mt, rr), base);
    }
    return a;
  };

  // ---- S^T = K Q^T (plus the accumulator start) for the sub-tile at key j0n in K slot SLOT
  auto qk = [&](auto slot_c, f32x16 (&s)[2], int j0n) {
    constexpr int SLOT = decltype(slot_c)::value;
    const uint8_t* kb = smem + SLOT * L::TILE;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = acc_start(j0n, mt);
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kb + kfrag(t) + mt * 32 * L::KROW);
        s[mt] = mfma32(__builtin_bit_cast(bf16x8, kv), qf[t], s[mt]);
      }
    }
  };

  // ---- mask (partial / ragged sub-tiles), score_mod, tile maximum and the lazy
  // online-softmax rescale; returns how the weights of the tile are formed
  auto prep = [&](f32x16 (&s)[2], bool part, bool masked, int j0, auto dslot_c) -> TileMode {
    constexpr int DSLOT = decltype(dslot_c)::value;
    const int32_t* dl = reinterpret_cast<const int32_t*>(smem + 4 * L::TILE + DSLOT * KT * 4);
    const int jl = j0 + 4 * half;   // key of element (mt=0, rr=0) in this lane
    bool empty_tile = false;        // no row of the wave allows a key of the sub-tile
    if (masked) {
      if constexpr (MK == MK_GENERIC) {
        // the program over the lane's 32 keys at once, one bit per element
        auto span = [&](int lo, int hi) -> uint32_t { return ge_bits(lo - jl) & ~ge_bits(hi - jl + 1); };
        uint32_t ok = span(0, kv_len - 1);
        if (part) {
          uint32_t db = 0;
          if (stage_doc) {
            // one 4-key group at a time (unrolled, the eight reads would be issued
            // together and hold 32 registers)
#pragma unroll 1
            for (int g = 0; g < 8; ++g) {   // g = 4 mt + g4
              const u32x4 dv = *reinterpret_cast<const u32x4*>(dl + 8 * g + 4 * half);
              uint32_t nib = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e) nib |= (int)dv[e] == doc_i ? 1u << e : 0u;
              db |= nib << (4 * g);
            }
          }
          ok &= mask_word(p.prog, [&](int op, int a) { return row_leaf(op, a, i_g, span, db); });
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) s[mt][rr] = (ok >> (16 * mt + rr)) & 1u ? s[mt][rr] : kNegInf;
      } else {
        // Keys outside the row's [lo, hi] (hi already clipped to kv_len - 1) are masked;
        // when only the ragged tail needs masking the same test applies with the tail
        // bound alone.  The sub-tile is first decided for the whole wave: every row
        // allowing every key (nothing to mask), no row allowing any key (no weights), or
        // a test per element, which compares documents only when the sub-tile's keys
        // belong to more than one document.
        static_assert(KT == 64, "one key of the sub-tile per lane");
        uint32_t lo_t = lo_u, span_t = span;
        if (!part) {
          lo_t = 0;
          span_t = (uint32_t)(kv_len - 1);
        }
        const uint32_t ju = (uint32_t)j0;
        const uint32_t hi_t = lo_t + span_t;
        bool all_in = lo_t <= ju && ju + (KT - 1) <= hi_t;
        bool none_in = hi_t < ju || lo_t > ju + (KT - 1);
        bool key_docs = false;
        if constexpr (kDoc) {
          if (part) {
            const int dk = dl[lane];   // document of key j0 + lane
            const int dt = __builtin_amdgcn_readfirstlane(dk);
            if (__ballot(dk != dt) != 0) {
              key_docs = true;
              all_in = false;
            } else if (dt != doc_i) {   // one document, not the row's: nothing allowed
              all_in = false;
              none_in = true;
              lo_t = 0x80000000u;
              span_t = 0;
            }
          }
        }
        if (__ballot(!all_in) == 0) {
          masked = false;
        } else if (__ballot(!none_in) == 0) {
          masked = false;
          empty_tile = true;
        } else {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              int dq[4] = {doc_i, doc_i, doc_i, doc_i};
              if constexpr (kDoc) {
                if (key_docs) {
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
                s[mt][rr] = ok ? s[mt][rr] : kNegInf;
              }
            }
        }
      }
    }

    // Monotone kinds keep the raw score (the tile maximum is mapped once); the others
    // store t = log2(e) * score_mod(s * scale) (-inf stays -inf).
    bool raw;
    float bias2 = 0.f;  // constant base-2 bias of a saturated relative-position tile
    if constexpr (SCORE == FA_S_IDENTITY) {
      raw = true;
    } else if constexpr (SCORE == FA_S_SOFTCAP) {
      raw = true;   // monotone: the maximum is taken on raw scores
    } else if constexpr (SCORE == FA_S_RELPOS) {
      const int dmin = i_wave0 - (j0 + KT - 1);
      const int dmax = i_wave0 + 31 - j0;
      raw = dmin >= R || dmax <= -R;
      bias2 = dmin >= R ? bias_far2 : bias_ahead2;
      if (!raw) {
        // stored in natural units, s * scale + table[i - j] (mapped to base 2 with the
        // tile maximum and in the weights).  The lane's entries sit at fixed offsets
        // below the entry of its last key, in the padded table or in the K slot's window.
        constexpr int kLast = key_of(1, 15);
        const int dd_last = i_g - (jl + kLast);
        const float* tb = rel_in_lds ? rel_lds + (dd_last + R + kRelPad)
                                     : rel_lds + (DSLOT * kRelWin + dd_last - (i_wg0 - j0 - (KT - 1)));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            s[mt][rr] = __builtin_fmaf(s[mt][rr], p.scale, tb[kLast - key_of(mt, rr)]);
      }
    } else {
      raw = true;   // ALiBi: the bias is already in the accumulator (acc_start)
    }
    // the maximum of this lane's half of the row's tile (16 of the 32 keys per 32-key
    // tile; the other half lives in lane ^ 32); not needed with a fixed reference
    float tmax = kNegInf;
    if (!fixed_ref && !empty_tile) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, s[mt][rr]);
    }
    // map a raw-score maximum into the base-2 domain
    auto to_base2 = [&](float t) -> float {
      if (raw && t != kNegInf) {
        if constexpr (SCORE == FA_S_SOFTCAP) {
          return sc.cap2 - 2.f * sc.cap2 * fast_rcp(fast_exp2(t * sc.capk) + 1.f);
        } else {
          return __builtin_fmaf(t, sc.c2, bias2);
        }
      }
      if constexpr (SCORE == FA_S_RELPOS) return t * kLog2e;   // natural units (-inf stays)
      return t;
    };
    // lazy rescale (wave-uniform branch): the reference moves only when a row's tile
    // maximum exceeds it by more than kRescaleThresh.  A row's maximum exceeds it iff one
    // of its halves does, so the exchange between the halves (an LDS round trip) is
    // needed only inside the rare rescale branch.
    if (!fixed_ref && __ballot(to_base2(tmax) > m_run + kRescaleThresh) != 0) {
      const float m_cand = to_base2(fmaxf(tmax, __shfl_xor(tmax, 32)));
      const bool grow = m_cand > m_run + kRescaleThresh;
      const float m_new = grow ? m_cand : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;   // 0 when m_run = -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    TileMode md;
    md.one = 1.f;
    if constexpr (SCORE == FA_S_SOFTCAP) {
      md.mul = 0.f;
      md.add = sc.cap2 - m_use;
      if (masked) {
        // y = log2(exp2(s capk) + 1) / capk keeps -inf and reproduces the weight with one = 0
        const float inv_k = 1.f / sc.capk;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float x = s[mt][rr];
            const float y = fast_log2(fast_exp2(x * sc.capk) + 1.f) * inv_k;
            s[mt][rr] = (x == kNegInf) ? kNegInf : y;
          }
        md.one = 0.f;
      }
    } else if (raw) {
      md.mul = sc.c2;
      md.add = bias2 - m_use;
    } else {
      md.mul = SCORE == FA_S_RELPOS ? kLog2e : 1.f;
      md.add = -m_use;
    }
    if (empty_tile) md.add = kNegInf;   // every weight of the sub-tile is exactly zero
    return md;
  };

  // ---- one pipelined step: the weights P of the tile in s (bf16 pairs), O^T += V^T P^T
  // with V from V slot VS, and (QK) the scores of the next tile into sn from K slot KS.
  // Five groups, fenced for the scheduler: group g reads V of 16-key step g-1 and K of
  // quarter g of the next QK product, forms P of step g (VALU that covers the LDS
  // latency), then multiplies P of step g-1 with V and runs QK quarter g; no MFMA of a
  // group waits on VALU of the same group.
  auto fused = [&](auto vs_c, auto ks_c, const f32x16 (&s)[2], f32x16 (&sn)[2],
                   const TileMode& md, auto qk_c, int jn) -> float {
    constexpr int VS = decltype(vs_c)::value;
    constexpr int KS = decltype(ks_c)::value;
    constexpr bool QK = decltype(qk_c)::value;   // the last step of a pass has no next tile
    constexpr int KQ = KSTEPS / 2;   // k-steps per quarter of the QK product
    const uint8_t* vb = smem + (2 + VS) * L::TILE;
    const uint8_t* kb = smem + KS * L::TILE;
    float psum = 0.f;
    u32x4 kf[KQ];
    bf16x8 vf[DM];
    u32x4 pk[2];
    auto read_k = [&](auto q_c, u32x4 (&dst)[KQ]) {
      constexpr int q = decltype(q_c)::value;
#pragma unroll
      for (int i = 0; i < KQ; ++i) {
        const int t = (q & 1) * KQ + i;
        dst[i] = *reinterpret_cast<const u32x4*>(kb + kfrag(t) + (q >> 1) * 32 * L::KROW);
      }
    };
    auto read_v = [&](auto t_c, bf16x8 (&dst)[DM]) {
      constexpr int t = decltype(t_c)::value;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const uint8_t* va = vb + vaddr[dm] + 16 * t * L::KROW;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(va + 8 * L::KROW));
        dst[dm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto p_step = [&](auto t_c, u32x4& dst) {
      constexpr int t = decltype(t_c)::value;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float pv2[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float x = s[t >> 1][8 * (t & 1) + 2 * e2 + h2];
          float arg;
          if constexpr (SCORE == FA_S_SOFTCAP) {
            const float rr = fast_rcp(fast_exp2(x * sc.capk) + md.one);
            arg = __builtin_fmaf(-2.f * sc.cap2, rr, md.add);
          } else {
            arg = __builtin_fmaf(x, md.mul, md.add);
          }
          pv2[h2] = fast_exp2(arg);
        }
        dst[e2] = cvt_pk_bf16(pv2[0], pv2[1]);
        psum += pv2[0] + pv2[1];
      }
    };
    // The fragments of each group are read one group ahead, right after the MFMAs that
    // consumed the previous ones were issued, so their LDS latency runs under those
    // MFMAs; only group 0's K quarter is read at entry, where the weights of 16-key
    // step 0 (VALU) cover it.
    if constexpr (QK) read_k(std::integral_constant<int, 0>{}, kf);
    __builtin_amdgcn_sched_barrier(0);
    static_for<5>([&](auto g_c) {
      constexpr int g = decltype(g_c)::value;
      if constexpr (g < 4) p_step(g_c, pk[g & 1]);
      if constexpr (g >= 1) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[(g - 1) & 1]);
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) oacc[dm] = mfma32(vf[dm], pb, oacc[dm]);
      }
      if constexpr (QK && g < 4) {
        constexpr int mt = g >> 1;
        if constexpr ((g & 1) == 0) sn[mt] = acc_start(jn, mt);
#pragma unroll
        for (int i = 0; i < KQ; ++i)
          sn[mt] = mfma32(__builtin_bit_cast(bf16x8, kf[i]), qf[(g & 1) * KQ + i], sn[mt]);
      }
      if constexpr (g < 4) read_v(g_c, vf);
      if constexpr (QK && g + 1 < 4) read_k(std::integral_constant<int, g + 1>{}, kf);
      __builtin_amdgcn_sched_barrier(0);
    });
    return psum;
  };

  // ---- the row's block list (full entries, then partial) in passes of kListCap entries.
  // Software pipeline over sub-tiles: while the weights of sub-tile s are formed and
  // multiplied with V_s, the scores of s+1 are computed from K_{s+1}; K runs one sub-tile
  // ahead of V in the copies (K_{s+2} and V_{s+1} are in flight during step s).
  const cptr flist_c = (cptr)sreg(flist), plist_c = (cptr)sreg(plist);
  for (int c0 = 0; c0 < n_ent; c0 += kListCap) {
    const int cnt = min(kListCap, n_ent - c0);
    const int nsub = cnt << spb_sh;
    // prologue: K_0, V_0 (and K_1) resident, scores of sub-tile 0 prepared.  The first
    // tiles' positions come from scalar loads of the list, so their copies go out
    // before the list is staged in LDS and the two round trips overlap.
    auto ent = [&](int e) -> int { return c0 + e < nf ? flist_c[c0 + e] : plist_c[c0 + e - nf]; };
    int j0_a = ent(0) * bk;                                                  // sub-tile s
    int j0_b = nsub > 1 ? ent(1 >> spb_sh) * bk + (1 & spb_sh) * KT : 0;     // sub-tile s + 1
    copy_op(j0_a, std::false_type{}, std::integral_constant<int, 0>{});
    copy_op(j0_a, std::true_type{}, std::integral_constant<int, 0>{});
    if (nsub > 1) copy_op(j0_b, std::false_type{}, std::integral_constant<int, 1>{});
    for (int e = tid; e < cnt; e += NT) {
      const int ge = c0 + e;
      list_s[e] = ge < nf ? flist[ge] : plist[ge - nf];
    }
    // the list entry of the K copy of the next step, read one step ahead and kept as the
    // raw LDS value, so that no step starts with an LDS round trip (it also gives the
    // next step's tile start without another read)
    auto raw_ent = [&](int s) -> int { return list_s[s >> spb_sh]; };
    int kpos_raw = 0;
    auto sub_part = [&](int s) -> bool { return c0 + (s >> spb_sh) >= nf; };
    wait_dma();
    if (c0 == 0) {
      // consume Q and the row's document ID now that every load of the prologue has
      // landed: the tile copies are invisible to the compiler's wait counting, so a
      // load still counted as pending inside the tile loop would make its uses wait
      // for all memory, copies in flight included
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) asm volatile("" : "+v"(qf[t]));
      asm volatile("" : "+v"(doc_i));
    }
    __syncthreads();
    f32x16 sa[2], sb[2];
    qk(std::integral_constant<int, 0>{}, sa, j0_a);
    TileMode md = prep(sa, sub_part(0), sub_part(0) || j0_a + KT > kv_len, j0_a, std::integral_constant<int, 0>{});
    // step 0 refills K slot 0 (with its document-ID and position-window slots), which
    // every wave has just read above
    if (nsub > 2) __syncthreads();
    kpos_raw = nsub > 2 ? raw_ent(2) : 0;

    // step s (slot parity P = s & 1): V_s in V slot P, K_{s+1} in K slot 1-P; copies of
    // K_{s+2} into K slot P and V_{s+1} into V slot 1-P
    auto step = [&](int s, auto par_c, f32x16 (&scur)[2], f32x16 (&snxt)[2]) {
      constexpr int P = decltype(par_c)::value;
      using SP = std::integral_constant<int, P>;
      using SQ = std::integral_constant<int, 1 - P>;
      const bool more = s + 1 < nsub;
      if (s + 2 < nsub) copy_op(uniform(kpos_raw) * bk + ((s + 2) & spb_sh) * KT, std::false_type{}, SP{});
      if (more) copy_op(j0_b, std::true_type{}, SQ{});
      // the last step of a pass also multiplies the (stale) other K slot: its scores are
      // discarded.  A second copy of the step without that product makes the register
      // allocator spill (about 250-470 bytes per lane), which costs far more than the
      // 16 MFMAs per pass it saves.
      l_run += fused(SP{}, SQ{}, scur, snxt, md, std::true_type{}, j0_b);
      if (more) {
        const bool part = sub_part(s + 1);
        md = prep(snxt, part, part || j0_b + KT > kv_len, j0_b, SQ{});
        j0_a = j0_b;
        j0_b = s + 2 < nsub ? uniform(kpos_raw) * bk + ((s + 2) & spb_sh) * KT : 0;
      }
      kpos_raw = s + 3 < nsub ? raw_ent(s + 3) : 0;
      wait_dma();
      __syncthreads();
    };
    for (int s = 0; s < nsub; s += 2) {
      step(s, std::integral_constant<int, 0>{}, sa, sb);
      if (s + 1 < nsub) step(s + 1, std::integral_constant<int, 1>{}, sb, sa);
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
