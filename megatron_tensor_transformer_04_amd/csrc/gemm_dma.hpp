// Direct-to-LDS MFMA GEMM engine for gfx950: C[M][N] = sum_k P[m][k] Q[k][n]
// with 16-bit operands and fp32 accumulation in v_mfma_f32_32x32x16_{f16,bf16}.
//
// This is the engine for large tiles. Operand tiles travel from HBM/L2
// straight into LDS with buffer_load_dwordx4 ... lds: no VGPRs hold staged
// data, no ds_write is issued, and rows or k-chunks outside the matrix are
// zero-filled by the buffer unit's range check (num_records) instead of by
// branches.
//
// Operand layouts. Each operand is either k-contiguous ("KC": P[m][k] at
// p[m*ld + k], Q[k][n] at q[n*ld + k]) or mn-contiguous ("MC": P[m][k] at
// p[k*ld + m], Q[k][n] at q[k*ld + n]).
//
// LDS holds two stages of one k-tile (BK deep) each, P's tile then Q's,
// each stage its own array: [P stage 0][Q stage 0], [P stage 1][Q stage 1].
//   KC tile: [rows][BK], rows of BK/8 16-byte chunks; chunk c of row r sits
//            at c ^ sk(r): sk(r) = (r & 7) ^ ((r >> 3) & 1) for BK = 64,
//            ((r >> 1) ^ (r >> 3)) & 3 for BK = 32; in the 16x16 form
//            (below) rot(r & 7) ^ (4 ((r >> 3) & 1)), rot = the three bits
//            rotated right by one.
//   MC tile: [BK][R], k-rows of R/16 32-byte units; unit u of k-row k sits
//            at u ^ sm(k), sm(k) = (k & 3) ^ ((k & 3) << 1) (mod 8), in the
//            16x16 form sm(k) ^ 4 ((k >> 3) & 1).
// A fragment read by 8 or 16 consecutive lanes (KC, ds_read_b128) and by 16
// or 32 consecutive lanes (MC, ds_read_b64_tr_b16) touches distinct banks
// under either swizzle, and both depend only on the lane, so every fragment
// of a wave is addressed as a per-lane base register plus an immediate. The
// 16x16 form's reads (16 consecutive rows, one chunk each) meet in the
// banks under sk: rows r and r + 2 are 64 banks apart, so the eight rows of
// one parity need eight distinct chunks, which rot(r & 7) ^ 4 ((r >> 3) & 1)
// gives and (r & 7) ^ ((r >> 3) & 1) does not (measured on MI355X: about
// 250x fewer LDS bank-conflict cycles, 1.5x the read rate).
//
// A direct LDS load writes the 16 bytes of lane l at offset 16 l of a 1 KB
// block, so the swizzle is applied on the global side: lane l fetches the
// logical chunk that belongs at its fixed LDS slot.
//
// MFMA: v_mfma_f32_32x32x16_{bf16,f16}. Lane l supplies row (A) / column (B)
// l % 32 and the eight k values 8 (l / 32) .. 8 (l / 32) + 7, and holds the
// results C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r = 0..15. A fragment
// comes from a KC tile with one ds_read_b128 and from an MC tile with two
// ds_read_b64_tr_b16 transposing reads.
//
// The 16x16 form (DmaTile MF16; KC operands, BK = 64, a plain or bias + GeLU
// store): v_mfma_f32_16x16x32_{bf16,f16}, lane l supplies row / column l % 16
// and k values 8 (l / 16) .. + 7 of a 32-wide substep and holds
// C[4 (l / 16) + r][l % 16], r = 0..3. Same tiles, same k order per
// element (on MI355X the outputs of 16384 x 10240 x 10240 matched the 32x32
// form's bit for bit); the chip holds a higher clock under this form (1.56
// against 1.40 GHz under the profiler with 256 x 320 tiles, for 2.6 % less
// time in plain runs). Its fragments fill more registers per flop (a 64 x
// 160 wave tile: 40 of 16x16 against 10 of 32x32, the same accumulator
// bytes but 14 reads of 16 B per 32-wide substep instead of 7 per 16), so
// one set of fragment registers serves both substeps: each is refilled as
// soon as its last MFMA of the substep has issued (see the k-loop).
//
// Pipeline. Within one output tile, k-tile t lives in stage t % 2 (tiles
// run in pairs, so that each access names its stage's array at compile
// time) and is consumed in BK/16 substeps (fragments double-buffered in
// registers). Tiles 0 and 1 are issued first; iteration t (BK = 64, four
// substeps) then does
//   read frags (t, 1)        | MFMAs (t, 0)
//   read frags (t, 2)        | MFMAs (t, 1)
//   read frags (t, 3)
//   -- wait until tile t+1 has landed (later tiles may still be in flight),
//      barrier: every wave is done with stage t % 2 --
//   first half of the loads of tile t+2 into stage t % 2 | MFMAs (t, 2)
//   rest of those loads, read frags (t+1, 0)              | MFMAs (t, 3)
// so LDS reads overlap MFMAs and a tile's global loads have about one
// iteration of MFMA work to land. Placing the barrier one substep before
// the end of the tile spreads each wave's loads over 20 MFMAs instead of
// 10: issued in one burst after the barrier, the loads of all eight waves
// filled the texture unit's queues and stalled the MFMAs interleaved with
// them (measured on MI355X with the SQ_VMEM_TA_*_FIFO_FULL counters).
// Scheduling constraints hold this order (the compiler's own schedule
// serialises each read with its first use); the reads and, after the
// barrier, the loads are interleaved one by one with the MFMAs. Workgroups are
// persistent (see gemm_dma_kernel): the next output tile's k-tile 0 is
// issued before the current tile's epilogue.
//
// Workgroup -> tile order: see map_work and tile_coords.
#pragma once

#include <type_traits>

#include "gemm_mfma.hpp"

namespace tpmlp {

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// OCC_: workgroups per CU the tile is built for (their waves share each
// SIMD's registers and the CU's LDS). MF16_: the 16x16x32 MFMA form (see
// the header comment; k-contiguous operands, 64-deep k-tiles).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_, int OCC_ = 1, bool MF16_ = false>
struct DmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, OCC = OCC_;
  static constexpr bool MF16 = MF16_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES = WAVES_M_ * WAVES_N_;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FRAG = MF16 ? 16 : 32;  // fragment edge
  static constexpr int FM = WTM / FRAG, FN = WTN / FRAG;
  static constexpr int LDS_P = BM * BK * 2, LDS_Q = BN * BK * 2;  // one stage of P / Q
  static constexpr int STG = LDS_P + LDS_Q;                       // one stage (P, then Q)
  static constexpr int LDS_BYTES = STAGES * STG;
  // direct loads (1 KB blocks) per wave per stage
  static constexpr int LP = LDS_P / 1024 / WAVES, LQ = LDS_Q / 1024 / WAVES;
  static constexpr int GROUP = 8;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(LP * WAVES * 1024 == LDS_P && LQ * WAVES * 1024 == LDS_Q, "tile not divisible into 1 KB blocks");
  static_assert(BM >= 128 && BN >= 128 && BM <= 512 && BN <= 512, "MC tiles need 8..32 32-byte units per k-row");
  static_assert(STAGES >= 2, "at least two stages");
  static_assert(BK == 32 || BK == 64, "k-tiles of 32 or 64 (an even number of 16-wide substeps)");
  static_assert(BK == 32 || WAVES % 2 == 0, "64-deep KC tiles need an even number of waves");
  // 16x16 form: one set of fragment registers refilled as it is consumed
  // (ROLLED, see the k-loop) where two sets and the accumulators would pass
  // 224 of the 256 registers a lane has at two waves per SIMD.
  static constexpr bool ROLLED = MF16 && (FM + FN) * 2 * 4 + FM * FN * 4 > 224;
  static_assert(!MF16 || BK == 64, "16x16 form: two 32-wide substeps per k-tile");
  static_assert(!ROLLED || LP + LQ <= FN - 1, "rolled 16x16 form: one load per column");
  static_assert(LDS_BYTES * OCC <= 160 * 1024, "LDS is 160 KB per CU");
  static constexpr int WAVES_PER_SIMD = WAVES * OCC / 4;
  static constexpr int PER_XCD = 32 * OCC;  // workgroups in flight per XCD
};

// s_waitcnt immediate (gfx9 encoding) that waits until at most N vector
// memory operations of this wave are outstanding: vmcnt in bits 3:0 and
// 15:14, expcnt (bits 6:4) and lgkmcnt (bits 11:8) left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt 0), not for its direct-to-LDS loads. __syncthreads' fence would
// also wait for every outstanding direct load (their LDS writes count as
// prior stores), which removes the overlap the loads are issued early for;
// callers wait for the loads they need with wait_vmcnt. The asm statement's
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0; vmcnt (63) and expcnt (7) at their maxima
  asm volatile("s_barrier" ::: "memory");
}

// Instruction-order constraints for the machine scheduler (AMDGPU
// sched_barrier / sched_group_barrier masks: 0x008 MFMA, 0x020 VMEM read,
// 0x100 DS read). sched_fence: nothing moves across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// The region just ended issues MF MFMAs, VM vector-memory reads and DS DS
// reads: order them as MFMA, VMEM, DS, DS.., MFMA, DS.. (one VMEM after every
// MF / VM-th MFMA, up to ceil(DS / MF) DS reads after each) and close the
// region.
template <int MF, int VM, int DS>
__device__ __forceinline__ void sched_interleave() {
  constexpr int DPER = (DS + MF - 1) / MF;
  constexpr int VS = VM > 0 && MF / VM > 1 ? MF / VM : 1;  // MFMAs per VMEM read
  static_for<0, MF>([&](auto i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (i % VS == 0 && i / VS < VM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    constexpr int d = DS - i * DPER < DPER ? DS - i * DPER : DPER;
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);
  });
  sched_fence();
}

// The 16x16 form's substep (see the k-loop): NB - 1 columns of FMA MFMAs,
// each followed by one VMEM read (the first VM columns) and one DS read,
// then the last column one MFMA and one DS read at a time, then one DS read.
template <int NB, int FMA, int VM>
__device__ __forceinline__ void sched_rolling() {
  static_for<0, NB - 1>([&](auto j) {
    __builtin_amdgcn_sched_group_barrier(0x008, FMA, 0);
    if constexpr (j < VM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  });
  static_for<0, FMA>([&](auto i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  });
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  sched_fence();
}

// Opaque copies: the compiler can neither hoist out of a loop nor merge what
// is computed from the result. The constraints are AMDGPU register classes
// (v: VGPR, s: SGPR), so the statements exist in the device pass only.
__device__ __forceinline__ int opaque_v(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
}
__device__ __forceinline__ int opaque_s(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+s"(x));
#endif
  return x;
}

// Offsets beyond every buffer's num_records: the load returns zeros.
constexpr uint32_t kOobOffset = 0x80000000u;

template <int BK, bool MF16 = false>
__device__ __forceinline__ int dsk(int r) {
  if constexpr (MF16) {  // BK = 64: the low three row bits rotated right, bit 2 flipped on odd 8-row groups
    const int lo = r & 7;
    return (((lo & 1) << 2) | (lo >> 1)) ^ (((r >> 3) & 1) << 2);
  }
  if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);
  return ((r >> 1) ^ (r >> 3)) & 3;
}

template <bool MF16 = false>
__device__ __forceinline__ int dsm(int k) {
  const int s = ((k & 3) ^ ((k & 3) << 1)) & 7;
  return MF16 ? s ^ (((k >> 3) & 1) << 2) : s;  // 16x16 form: k-row bit 3 flips bit 2
}

// Workgroup -> work order for kernels that run one workgroup per CU. The
// hardware hands workgroup b to XCD b % 8, and each XCD has its own L2;
// all XCDs share the memory-side cache (MALL). Each "wave" of 8 x PER
// consecutive work items (PER = workgroups in flight per XCD) is split into
// 8 runs of PER, one per XCD. Tiles are numbered GROUP tile-rows at a time,
// column-major inside a group (tile_coords), so the tiles in flight on one
// XCD form a compact GROUP x PER/GROUP block (L2 reuse of both operand
// panels) and the eight XCDs work side by side on the same row panels (MALL
// reuse across XCDs). A last partial wave keeps the plain order.
template <int PER>
__device__ __forceinline__ int map_work(int b, int nblk) {
  constexpr int WAVE = 8 * PER;
  if (b < nblk / WAVE * WAVE) {
    const int x = b & 7, p = b >> 3;
    return (p / PER) * WAVE + x * PER + p % PER;
  }
  return b;
}

template <int GROUP>
__host__ __device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int gid = t / (GROUP * tiles_n);
  const int first = gid * GROUP;
  const int gsz = min(tiles_m - first, GROUP);
  const int in = t - gid * GROUP * tiles_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

// Work items past the last full wave of tiles. With T tiles and W workgroups
// per wave, a last wave of r = T % W tiles would leave most CUs idle; when
// parts > 1 those r tiles are instead each split into `parts` k-ranges of
// k_part (a multiple of the k-tile), one work item each, whose fp32 partial
// sums go to `partial` ([r][parts][BM][BN]) and are added, in part order, by
// tail_finish_kernel. Work item w < full is tile w over all of K.
struct TailSplit {
  int full;       // tiles computed whole
  int parts;      // k-ranges per tail tile (1: no tail split)
  int64_t k_part; // k elements per range
  float* partial;
};

// The second GEMM of a paired launch (gemm_dma_kernel's PAIR form): its
// operands and epilogue; shape, pitches and layout are the first one's.
// tiles: the tile count of each GEMM.
template <class Epi>
struct PairGemm {
  const uint16_t* p;
  const uint16_t* q;
  Epi epi;
  int tiles;
};

// Raw buffer resource (stride 0) over `bytes` bytes at `p`, built from
// wave-uniform values so that it lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes < 0x7fffffff ? bytes : 0x7fffffff));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, n, 0x00020000);
}

// Source of the 16 bytes that lane `lane` writes in 1 KB block `blk` of an
// operand tile: element offset from the tile origin at k = 0 (`rel`), the
// tile-local row (KC) or column (MC) index `mn`, and the k offset `kk`.
template <bool KC, int R, int BK, bool MF16 = false>
__device__ __forceinline__ void dma_slot(int blk, int lane, int64_t ld, int64_t& rel, int& mn, int& kk) {
  if constexpr (KC) {
    constexpr int CH = BK / 8;                // 16-byte chunks per row
    const int r = blk * (64 / CH) + lane / CH;  // 1024 / (2 BK) rows per block
    const int kc = (lane % CH) ^ dsk<BK, MF16>(r);
    mn = r;
    kk = kc * 8;
    rel = (int64_t)r * ld + kk;
  } else {
    const int o = blk * 1024 + lane * 16;
    const int kr = o / (R * 2), w = o % (R * 2);
    const int u = (w >> 5) ^ dsm<MF16>(kr);
    const int c8 = 2 * u + ((w >> 4) & 1);
    mn = c8 * 8;
    kk = kr;
    rel = (int64_t)kr * ld + mn;
  }
}

// k offset of direct load c's chunk relative to load 0's (same lane). KC:
// the chunk's k depends on the row only through r & 15, and load c's rows
// are c * WAVES * 1024 / (2 BK) further on: a multiple of 16 (for BK = 64
// because WAVES is even). MC: each load covers 1024 / (2R) k-rows.
template <bool KC, int R, int WAVES>
__host__ __device__ constexpr int dma_kstep(int c) {
  return KC ? 0 : c * WAVES * (1024 / (2 * R));
}

// Per-lane LDS byte offsets of a wave's MFMA fragments (relative to a
// stage's array; every stage uses the same offsets). NF fragments of
// 32 rows (KC) or 32 columns (MC), the first at tile row / column `first`
// (a multiple of 32).
template <bool KC, int R, int BK, int NF>
struct FragAddr {
  static constexpr int NB = KC ? BK / 16 : NF;
  uint32_t base[NB];

  __device__ __forceinline__ void init(int lane, int region, int first) {
    if constexpr (KC) {
      // row first + 32 i + (l & 31); 16-byte chunk 2 ks + (l >> 5)
      const int r = lane & 31;
#pragma unroll
      for (int ks = 0; ks < NB; ++ks)
        base[ks] = (uint32_t)(region + (first + r) * (2 * BK) + (((2 * ks + (lane >> 5)) ^ dsk<BK>(r)) << 4));
    } else {
      // lanes 16 G .. 16 G + 15: 32-byte unit first/16 + 2 i + (G & 1),
      // k-rows 16 ks + 8 (G >> 1) + 4 hh + (j >> 2), 8-byte piece j & 3
      const int G = lane >> 4, j = lane & 15;
      const int kr = 8 * (G >> 1) + (j >> 2);
      const int u0 = first >> 4;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        base[i] = (uint32_t)(region + kr * (R * 2) + (((u0 + 2 * i + (G & 1)) ^ dsm(kr)) << 5) + ((j & 3) << 3));
    }
  }


  // Fragment I for k-substep KS (16 wide) of the stage the bases point at.
  // Move every base by `delta` bytes (to the other stage of one array).
  __device__ __forceinline__ void advance(uint32_t delta) {
#pragma unroll
    for (int i = 0; i < NB; ++i) base[i] += delta;
  }
  template <int I, int KS>
  __device__ __forceinline__ u32x4 read(const char* lds) const {
    if constexpr (KC) {
      return *reinterpret_cast<const u32x4*>(lds + base[KS] + I * 32 * (2 * BK));
    } else {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      u32x4 out;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(lds + base[I] + (KS * 16 + hh * 4) * (R * 2)));
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        out[2 * hh] = w[0];
        out[2 * hh + 1] = w[1];
      }
      return out;
    }
  }
};

// Per-lane LDS byte offsets of a wave's 16x16x32 fragments (KC tiles with
// the MF16 swizzle, BK = 64): NF fragments of 16 rows, the first at tile row
// `first`. Lane l reads row first + 16 i + (l & 15), 16-byte chunk
// 4 ks + (l >> 4) of k-substep ks (32 wide).
template <int NF>
struct FragAddr16 {
  static constexpr int BK = 64, NB = 2;
  uint32_t base[NB];
  __device__ __forceinline__ void init(int lane, int region, int first) {
    const int r = lane & 15;
#pragma unroll
    for (int ks = 0; ks < NB; ++ks)
      base[ks] = (uint32_t)(region + (first + r) * (2 * BK) + (((4 * ks + (lane >> 4)) ^ dsk<BK, true>(r)) << 4));
  }
  // Move every base by `delta` bytes (to the other stage of one array).
  __device__ __forceinline__ void advance(uint32_t delta) {
#pragma unroll
    for (int i = 0; i < NB; ++i) base[i] += delta;
  }
  template <int I, int KS>
  __device__ __forceinline__ u32x4 read(const char* lds) const {
    return *reinterpret_cast<const u32x4*>(lds + base[KS] + I * 16 * (2 * BK));
  }
};

// The same for an MC tile [BK][R] (16x16 form swizzle): NF fragments of 16
// columns, the first at tile column `first` (a multiple of 16). Lanes 16 G
// .. 16 G + 15 read 32-byte unit first/16 + i, k-rows 32 ks + 8 G + 4 hh +
// (l % 16) / 4 (hh = 0, 1: two transposing reads), 8-byte piece l % 4: lane
// l gets column l % 16's eight k values 32 ks + 8 G .. + 7. Bits 0, 1 and 3
// of the k-row pick the unit's place, so the 32 lanes of groups 0 and 1
// touch 8 distinct places (all 64 banks).
template <int R, int NF>
struct FragAddrMC16 {
  static constexpr int NB = NF;
  uint32_t base[NB];
  __device__ __forceinline__ void init(int lane, int region, int first) {
    const int G = lane >> 4, j = lane & 15;
    const int kr = 8 * G + (j >> 2);
    const int u0 = first >> 4;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      base[i] = (uint32_t)(region + kr * (R * 2) + (((u0 + i) ^ dsm<true>(kr)) << 5) + ((j & 3) << 3));
  }
  // Move every base by `delta` bytes (to the other stage of one array).
  __device__ __forceinline__ void advance(uint32_t delta) {
#pragma unroll
    for (int i = 0; i < NB; ++i) base[i] += delta;
  }
  template <int I, int KS>
  __device__ __forceinline__ u32x4 read(const char* lds) const {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    u32x4 out;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const i16x4 v =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + base[I] + (KS * 32 + hh * 4) * (R * 2)));
      const u32x2 w = __builtin_bit_cast(u32x2, v);
      out[2 * hh] = w[0];
      out[2 * hh + 1] = w[1];
    }
    return out;
  }
};

// One workgroup per CU, each looping over work items v = blockIdx.x,
// blockIdx.x + gridDim.x, ... (nwork items: the tiles, with the tail tiles
// split into k-ranges, see TailSplit). Between two items the first k-tile
// of the next item is loaded into the free stage while the epilogue of the
// current one runs out of the other stage, so that its load latency hides
// behind the epilogue instead of stalling a freshly started workgroup.
//
// SLICED_P: P (k-contiguous) is read from the row slices xs; every slice
// holds a whole number of BM-row tiles (the host checks), so each work
// item's P tile lies in one slice and gets that slice's buffer resource.
//
// PAIR: two GEMMs of one shape, pitches and epilogue type in one launch
// (work items g2.tiles .. 2 g2.tiles - 1 are the second one's tiles, with
// g2's operands and epilogue), unsplit. Two launches of at most half a
// wave each then fill the CUs together, without the k-split's partials.
template <class Cfg, class S, bool P_KC, bool Q_KC, class Epi, bool SLICED_P = false, bool PAIR = false>
__global__ __launch_bounds__(Cfg::THREADS)
__attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_SIMD, Cfg::WAVES_PER_SIMD)))
void gemm_dma_kernel(GemmShape sh, Operand P, int64_t p_extent, Operand Q, int64_t q_extent, Epi epi_first,
                     TailSplit tail, int nwork, RowSlices xs, PairGemm<Epi> g2) {
  static_assert(!SLICED_P || P_KC, "row slices of a k-contiguous P only");
  static_assert(!(PAIR && SLICED_P), "a paired launch reads dense operands");
  // The epilogue of the item being finished (the second GEMM's for its
  // items in a paired launch).
  Epi epi = epi_first;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, LP = Cfg::LP, LQ = Cfg::LQ;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, ST = Cfg::STAGES, STG = Cfg::STG;
  constexpr bool M16 = Cfg::MF16;
  static_assert(!M16 || !Epi::kDirectF32, "16x16 form: a tile-wise epilogue");
  static_assert(!Cfg::ROLLED || (P_KC && Q_KC), "rolled 16x16 form: k-contiguous operands");
  static_assert((P_KC || (BM & (BM - 1)) == 0) && (Q_KC || (BN & (BN - 1)) == 0),
                "an mn-contiguous operand needs a power-of-two tile extent (swizzle, loads per k-row)");
  // The two stages are two LDS arrays, and every access names its array at
  // compile time (the k-loop runs tiles in pairs, tile t in stage t % 2):
  // the compiler then knows that a transposing fragment read of one stage
  // does not read what the direct loads in flight are writing into the
  // other. Through one array indexed at run time it waited for every
  // direct load in flight before each such read (the full load latency in
  // every k-tile of an mn-contiguous operand; ordinary LDS reads are not
  // affected).
  // Kernels without an mn-contiguous operand (no transposing reads) keep one
  // array, with the fragment offsets moved between the stages each tile:
  // two arrays cost them a second set of fragment address registers
  // (offsets past the 16-bit immediate), and their 16x16 forms spilled.
  static_assert(ST == 2, "two stages");
  constexpr bool TWO = !(P_KC && Q_KC) && !M16;
  static_assert(!(M16 && !(P_KC && Q_KC)), "the 16x16 form reads k-contiguous operands");
  __shared__ __attribute__((aligned(1024))) char ldsA[TWO ? STG : ST * STG];
  char* lds1 = ldsA + STG;
  if constexpr (TWO) {
    __shared__ __attribute__((aligned(1024))) char ldsB[STG];
    lds1 = ldsB;
  }
  char* const lds0 = ldsA;

  const int tid = threadIdx.x;
  int lane = tid & 63;  // made opaque at the top of every work item (see below)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

  // A work item: its output tile and k-range.
  struct Item {
    int tile, part;  // part >= 0: a k-range of a tail tile
    bool second;     // a tile of the second GEMM of a paired launch
    int tm, tn;
    int64_t m0, n0, kbeg;
    int kspan, nk;
  };
  auto decode = [&](int v) __attribute__((always_inline)) {
    Item it;
    int w = map_work<Cfg::PER_XCD>(v, nwork);
    it.second = false;
    if constexpr (PAIR) {
      it.second = w >= g2.tiles;
      if (it.second) w -= g2.tiles;
    }
    it.tile = w;
    it.part = -1;
    if (w >= tail.full) {
      it.tile = tail.full + (w - tail.full) / tail.parts;
      it.part = (w - tail.full) % tail.parts;
    }
    tile_coords<Cfg::GROUP>(it.tile, sh.tiles_m, sh.tiles_n, it.tm, it.tn);
    it.m0 = (int64_t)it.tm * BM;
    it.n0 = (int64_t)it.tn * BN;
    it.kbeg = it.part >= 0 ? (int64_t)it.part * tail.k_part : 0;
    const int64_t kend = it.part >= 0 ? min(sh.K, it.kbeg + tail.k_part) : sh.K;
    it.kspan = kend > it.kbeg ? (int)(kend - it.kbeg) : 0;
    it.nk = (it.kspan + BK - 1) / BK;
    return it;
  };
  // Buffer resources of an item's operand tiles, based at the tile origin
  // with num_records = the operand's extent from there, so any offset past
  // the tensor reads zeros. The 16x16 form also ends them at the matrix's
  // last row (its loads carry no per-row check).
  auto p_rsrc = [&](const Item& it) __attribute__((always_inline)) {
    if constexpr (SLICED_P) {
      const int64_t sl = it.m0 / xs.rows, r0 = it.m0 - sl * xs.rows;
      const int64_t rows = M16 ? min(xs.rows - r0, sh.M - it.m0) : xs.rows - r0;
      return uniform_rsrc(xs.p[sl] + r0 * P.ld, rows * P.ld * 2);
    } else {
      const int64_t base = P_KC ? it.m0 * P.ld : it.m0;
      const uint16_t* const ptr = PAIR && it.second ? g2.p : P.ptr;
      return uniform_rsrc(ptr + base,
                          (M16 && P_KC ? min(p_extent - base, (sh.M - it.m0) * P.ld) : p_extent - base) * 2);
    }
  };
  auto q_rsrc = [&](const Item& it) __attribute__((always_inline)) {
    const int64_t base = Q_KC ? it.n0 * Q.ld : it.n0;
    const uint16_t* const ptr = PAIR && it.second ? g2.q : Q.ptr;
    return uniform_rsrc(ptr + base,
                        (M16 && Q_KC ? min(q_extent - base, (sh.N - it.n0) * Q.ld) : q_extent - base) * 2);
  };

  // Per-lane byte offsets from the tile origin at k = 0; rows / columns
  // outside the matrix get kOobOffset. The k advance of each tile goes in
  // the instruction's scalar offset, so the K loop does no per-lane address
  // arithmetic. pk0 / qk0: the k offset (within a tile) of load 0's chunk
  // (the same for every item); load c's is that plus dma_kstep<>(c). The
  // 16x16 form keeps load 0's offset only (registers are short there): load
  // c's source is a fixed stride further on (KC: c * WAVES * 8 rows, with
  // the same chunk, as the swizzle depends on the row mod 16; MC: the
  // k-rows of dma_kstep<>(c), a multiple of 16, with the same columns). A KC
  // tile's rows past the matrix fall outside its buffer resource; an MC
  // tile's columns past the matrix read whatever lies there (inside the
  // buffer) or zeros (past it), and feed only output columns or rows past
  // the matrix, which no epilogue stores or sums.
  constexpr int NPV = M16 ? 1 : LP, NQV = M16 ? 1 : LQ;
  int pk0 = 0, qk0 = 0;
  auto offsets = [&](const Item& it, uint32_t(&pv)[NPV], uint32_t(&qv)[NQV]) __attribute__((always_inline)) {
    // Recomputed per item from an opaque copy of the lane index: hoisting
    // the item-independent 64-bit parts out of the item loop would keep
    // them live across the K loop.
    const int ln = opaque_v(lane);
    if constexpr (M16) {
      int64_t rel;
      int mn, kk;
      dma_slot<P_KC, BM, BK, true>(wave, ln, P.ld, rel, mn, kk);
      pv[0] = (uint32_t)rel * 2u;
      pk0 = kk;
      dma_slot<Q_KC, BN, BK, true>(wave, ln, Q.ld, rel, mn, kk);
      qv[0] = (uint32_t)rel * 2u;
      qk0 = kk;
      return;
    }
    static_for<0, NPV>([&](auto c) {
      int64_t rel;
      int mn, kk;
      dma_slot<P_KC, BM, BK>(c * Cfg::WAVES + wave, ln, P.ld, rel, mn, kk);
      pv[c] = it.m0 + mn < sh.M ? (uint32_t)rel * 2u : kOobOffset;
      if constexpr (c == 0) pk0 = kk;
    });
    static_for<0, NQV>([&](auto c) {
      int64_t rel;
      int mn, kk;
      dma_slot<Q_KC, BN, BK>(c * Cfg::WAVES + wave, ln, Q.ld, rel, mn, kk);
      qv[c] = it.n0 + mn < sh.N ? (uint32_t)rel * 2u : kOobOffset;
      if constexpr (c == 0) qk0 = kk;
    });
  };

  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int LOADS = LP + LQ;      // direct loads per wave per tile
  constexpr int FIRST = (LOADS + 1) / 2;  // loads in the first half (see the k-loop)
  // Direct loads of k-tile t of item `it` into stage `stage`: all of them
  // (PART 2), or the first FIRST (PART 0) or the rest (PART 1) in P-then-Q
  // order, or load PART - 3 alone (PART >= 3). On a K-tail tile, chunks at or beyond the item's k-range take
  // kOobOffset (one 32-bit compare per load); a tile past the end
  // (t >= nk) is all kOobOffset and fills its stage with zeros that nothing
  // reads, which keeps the loop body free of branches.
  auto issue_tile = [&](const Item& it, __amdgpu_buffer_rsrc_t prs, __amdgpu_buffer_rsrc_t qrs,
                        const uint32_t(&pv)[NPV], const uint32_t(&qv)[NQV], int t, char* const sp, auto part_c)
      __attribute__((always_inline)) {
    constexpr int PART = decltype(part_c)::value;
    const int krem = it.kspan - t * BK;  // k extent left from this tile on
    const int64_t k0 = krem > 0 ? it.kbeg + (int64_t)t * BK : 0;
    const int psoff = __builtin_amdgcn_readfirstlane((int)((P_KC ? k0 : k0 * P.ld) * 2));
    const int qsoff = __builtin_amdgcn_readfirstlane((int)((Q_KC ? k0 : k0 * Q.ld) * 2));
    if constexpr (M16) {
      // Load c's offset from load 0's (made opaque, so that the per-load
      // sums are formed here rather than kept in registers across the loop).
      // KC: all loads share load 0's k chunk, so one check against the
      // k-range selects kOobOffset for all (kOobOffset + c * step stays past
      // num_records); MC: load c's k-row is checked on its own.
      auto one = [&](__amdgpu_buffer_rsrc_t rs, uint32_t base, int k0c, int soff, bool kc, int64_t ld, int R,
                     int lds_off, auto c) __attribute__((always_inline)) {
        const int kstep = kc ? 0 : c * Cfg::WAVES * (1024 / (2 * R));
        const uint32_t step = kc ? (uint32_t)(Cfg::WAVES * 8 * ld * 2) : (uint32_t)(kstep * ld * 2);
        const uint32_t off = kc ? base + (uint32_t)c * step : (k0c + kstep < krem ? base + step : kOobOffset);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sp + lds_off + (c * Cfg::WAVES + wave) * 1024), 16,
                                                 off, soff, 0, 0);
      };
      const uint32_t pb = (uint32_t)opaque_v((int)(!P_KC || pk0 < krem ? pv[0] : kOobOffset));
      const uint32_t qb = (uint32_t)opaque_v((int)(!Q_KC || qk0 < krem ? qv[0] : kOobOffset));
      // PART >= 3: load PART - 3 alone (P's loads, then Q's)
      static_for<0, LP>([&](auto c) {
        if constexpr (PART == 2 || (PART < 2 && (PART == 0) == (c < FIRST)) || PART == 3 + c)
          one(prs, pb, pk0, psoff, P_KC, P.ld, BM, 0, c);
      });
      static_for<0, LQ>([&](auto c) {
        if constexpr (PART == 2 || (PART < 2 && (PART == 0) == (LP + c < FIRST)) || PART == 3 + LP + c)
          one(qrs, qb, qk0, qsoff, Q_KC, Q.ld, BN, Cfg::LDS_P, c);
      });
      return;
    }
    static_for<0, LP>([&](auto c) {
      if constexpr (PART == 2 || (PART < 2 && (PART == 0) == (c < FIRST)) || PART == 3 + c) {
        const uint32_t off = pk0 + dma_kstep<P_KC, BM, Cfg::WAVES>(c) < krem ? pv[c] : kOobOffset;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (lds_void*)(sp + (c * Cfg::WAVES + wave) * 1024), 16, off,
                                                 psoff, 0, 0);
      }
    });
    static_for<0, LQ>([&](auto c) {
      if constexpr (PART == 2 || (PART < 2 && (PART == 0) == (LP + c < FIRST)) || PART == 3 + LP + c) {
        const uint32_t off = qk0 + dma_kstep<Q_KC, BN, Cfg::WAVES>(c) < krem ? qv[c] : kOobOffset;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            qrs, (lds_void*)(sp + Cfg::LDS_P + (c * Cfg::WAVES + wave) * 1024), 16, off, qsoff, 0, 0);
      }
    });
  };
  constexpr auto kAll = std::integral_constant<int, 2>{};

  std::conditional_t<M16, std::conditional_t<P_KC, FragAddr16<FM>, FragAddrMC16<BM, FM>>, FragAddr<P_KC, BM, BK, FM>>
      pa;
  std::conditional_t<M16, std::conditional_t<Q_KC, FragAddr16<FN>, FragAddrMC16<BN, FN>>, FragAddr<Q_KC, BN, BK, FN>>
      qa;
  using AccT = std::conditional_t<M16, f32x4, f32x16>;
  AccT acc[FM][FN];
  u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto read_frags = [&](u32x4(&fa)[FM], u32x4(&fb)[FN], auto ks_c, const char* lds) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks_c)::value;
    static_for<0, FM>([&](auto i) { fa[i] = pa.template read<i, KS>(lds); });
    static_for<0, FN>([&](auto j) { fb[j] = qa.template read<j, KS>(lds); });
  };
  // Column-major over the wave's fragments: consecutive MFMAs share their B
  // fragment (measured on MI355X with the reads interleaved as below: about
  // 1.5 % faster than row-major on 16384 x 10240 x 10240).
  auto mfmas = [&](const u32x4(&fa)[FM], const u32x4(&fb)[FN]) __attribute__((always_inline)) {
    static_for<0, FN>([&](auto j) {
      static_for<0, FM>([&](auto i) {
        if constexpr (M16) acc[i][j] = S::mfma16x16x32(fa[i], fb[j], acc[i][j]);
        else acc[i][j] = S::mfma32x32x16(fa[i], fb[j], acc[i][j]);
      });
    });
  };
  // One substep's MFMAs (column-major) with, after MFMA k, a direct load
  // (loads L0 .. L0 + NL - 1, one after every (FM FN) / NL-th MFMA) and the
  // read of fragment k of substep KS into the other set (k < FM + FN, A
  // fragments first; none if KS < 0), in that program order. The
  // scheduling constraints alone did not keep the loads apart: the
  // compiler moved them all next to the barrier.
  auto mfmas_then = [&](const u32x4(&fa)[FM], const u32x4(&fb)[FN], u32x4(&na)[FM], u32x4(&nb)[FN], auto ks_c,
                        const char* lds, auto l0_c, auto nl_c, auto load) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks_c)::value, L0 = decltype(l0_c)::value, NL = decltype(nl_c)::value;
    static_for<0, FN>([&](auto j) {
      static_for<0, FM>([&](auto i) {
        if constexpr (M16) acc[i][j] = S::mfma16x16x32(fa[i], fb[j], acc[i][j]);
        else acc[i][j] = S::mfma32x32x16(fa[i], fb[j], acc[i][j]);
        constexpr int k = j * FM + i;
        constexpr int LS = NL > 0 && FM * FN / NL > 1 ? FM * FN / NL : 1;
        if constexpr (k % LS == 0 && k / LS < NL) load(std::integral_constant<int, 3 + L0 + k / LS>{});
        if constexpr (KS >= 0 && k < FM) na[k] = pa.template read<k, KS>(lds);
        else if constexpr (KS >= 0 && k >= FM && k < FM + FN) nb[k - FM] = qa.template read<k - FM, KS>(lds);
      });
    });
  };
  constexpr int NKS = BK / (M16 ? 32 : 16);  // substeps per k-tile
  // DS read instructions per substep (a transposing read moves half a
  // fragment).
  constexpr int DSR = (P_KC ? 1 : 2) * FM + (Q_KC ? 1 : 2) * FN;

  // Work item state is decoded again where it is needed rather than kept
  // live across the K loop (scalar registers are the scarce resource);
  // opaque_s() hides the work index from common-subexpression elimination.
  // Every item starts in stage 0: its tile count is rounded up to even.
  int v = blockIdx.x;
  {
    const Item first = decode(v);
    uint32_t pv[NPV], qv[NQV];
    offsets(first, pv, qv);
    issue_tile(first, p_rsrc(first), q_rsrc(first), pv, qv, 0, lds0, kAll);
  }
  while (true) {
    // Everything derived from the lane index is recomputed per item: hoisted
    // out of the item loop it would stay live across the K loop and the
    // epilogue and push the accumulators out of registers.
    lane = opaque_v(lane);
    const Item cur = decode(opaque_s(v));
    const __amdgpu_buffer_rsrc_t prs = p_rsrc(cur), qrs = q_rsrc(cur);
    uint32_t pv[NPV], qv[NQV];
    offsets(cur, pv, qv);
    issue_tile(cur, prs, qrs, pv, qv, 1, lds1, kAll);
    static_for<0, FM>([&](auto i) { static_for<0, FN>([&](auto j) { acc[i][j] = AccT{}; }); });
    pa.init(lane, 0, wm * Cfg::WTM);  // offsets within a stage
    qa.init(lane, Cfg::LDS_P, wn * Cfg::WTN);

    // One straight-line loop body: no branch at all, so the accumulators
    // keep their registers. The last iterations load and read stages
    // nothing uses again (in bounds; zeros or stale data, discarded).
    //
    // Software pipeline, pinned with scheduling constraints (left alone, the
    // compiler sinks each fragment read to just before its first MFMA and
    // exposes the full LDS latency on every read): the reads of substep s+1
    // are interleaved one by one with the MFMAs of substep s (one read after
    // each of the first MFMAs). After the barrier, the direct loads that
    // refill the freed stage and the reads of the next tile's first substep
    // are interleaved the same way with the MFMAs of the last substep.
    if (cur.nk > 0) {
      wait_vmcnt<(ST - 1) * LOADS>();  // k-tile 0 has landed
      barrier_lds();
      read_frags(fa0, fb0, std::integral_constant<int, 0>{}, TWO ? lds0 : ldsA);
      // k-tile t, in stage cs; tile t+1 is in stage ns, and tile t+2 goes
      // into cs once every wave has read tile t
      auto tile = [&](int t, char* const cs_, char* const ns_, uint32_t delta) __attribute__((always_inline)) {
        // fragment reads: the stage's array (two arrays), or the one array
        // with the offsets moved to tile t+1's stage after the barrier
        const char* const cs = TWO ? cs_ : ldsA;
        const char* const ns = TWO ? ns_ : ldsA;
        auto to_next = [&]() __attribute__((always_inline)) {
          if constexpr (!TWO) {
            pa.advance(delta);
            qa.advance(delta);
          }
        };
        if constexpr (Cfg::ROLLED) {
          // Two 32-wide substeps on one set of fragment registers: each B
          // fragment is refilled with the next substep's once its column of
          // MFMAs has issued, each A fragment once its last MFMA (in the
          // last column) has. Substep 0, then the barrier (this wave's reads
          // of tile t are all issued), then substep 1 with the loads that
          // refill the stage, one per column, and the reads of tile t+1.
          static_for<0, FN>([&](auto j) {
            static_for<0, FM>([&](auto i) {
              acc[i][j] = S::mfma16x16x32(fa0[i], fb0[j], acc[i][j]);
              if constexpr (j == FN - 1) fa0[i] = pa.template read<i, 1>(cs);
            });
            fb0[j] = qa.template read<j, 1>(cs);
          });
          sched_rolling<FN, FM, 0>();
          wait_vmcnt<(ST - 2) * LOADS>();
          barrier_lds();
          sched_fence();
          to_next();
          // the loads that refill stage cs, one after each column's MFMAs
          // (written in that order: left to the scheduler they bunched up
          // behind the first two columns)
          static_for<0, FN>([&](auto j) {
            static_for<0, FM>([&](auto i) {
              acc[i][j] = S::mfma16x16x32(fa0[i], fb0[j], acc[i][j]);
              if constexpr (j == FN - 1) fa0[i] = pa.template read<i, 0>(ns);
            });
            if constexpr (j < LOADS) issue_tile(cur, prs, qrs, pv, qv, t + ST, cs_, std::integral_constant<int, 3 + j>{});
            fb0[j] = qa.template read<j, 0>(ns);
          });
          sched_rolling<FN, FM, LOADS>();
        } else if constexpr (NKS >= 4) {
          // Substeps 0 .. NKS-3, then the reads of the last substep; with
          // those, this wave is done with stage cs and the barrier comes
          // one substep before the end of the tile: the loads that refill
          // the stage are spread over the last two substeps' MFMAs (half
          // each) instead of all landing on the texture unit at once.
          static_for<0, NKS - 2>([&](auto ks) {
            if constexpr (ks % 2 == 0) {
              read_frags(fa1, fb1, std::integral_constant<int, ks + 1>{}, cs);
              mfmas(fa0, fb0);
            } else {
              read_frags(fa0, fb0, std::integral_constant<int, ks + 1>{}, cs);
              mfmas(fa1, fb1);
            }
            sched_interleave<FM * FN, 0, DSR>();
          });
          read_frags(fa1, fb1, std::integral_constant<int, NKS - 1>{}, cs);  // NKS even: substep NKS-1 in set 1
          // Tile t+1 must have landed; tiles t+2 .. t+S-1 stay in flight.
          // The barrier also orders every wave's reads of tile t's stage
          // before the loads that refill it.
          wait_vmcnt<(ST - 2) * LOADS>();
          barrier_lds();
          sched_fence();
          to_next();
          auto load = [&](auto part) __attribute__((always_inline)) {
            issue_tile(cur, prs, qrs, pv, qv, t + ST, cs_, part);
          };
          // substep NKS-2 with the first FIRST loads
          mfmas_then(fa0, fb0, fa0, fb0, std::integral_constant<int, -1>{}, ns, std::integral_constant<int, 0>{},
                     std::integral_constant<int, FIRST>{}, load);
          sched_interleave<FM * FN, FIRST, 0>();
          // substep NKS-1 with the rest of the loads and tile t+1's first reads
          mfmas_then(fa1, fb1, fa0, fb0, std::integral_constant<int, 0>{}, ns, std::integral_constant<int, FIRST>{},
                     std::integral_constant<int, LOADS - FIRST>{}, load);
          sched_interleave<FM * FN, LOADS - FIRST, DSR>();
        } else {
          static_for<0, NKS - 1>([&](auto ks) {
            if constexpr (ks % 2 == 0) {
              read_frags(fa1, fb1, std::integral_constant<int, ks + 1>{}, cs);
              mfmas(fa0, fb0);
            } else {
              read_frags(fa0, fb0, std::integral_constant<int, ks + 1>{}, cs);
              mfmas(fa1, fb1);
            }
            sched_interleave<FM * FN, 0, DSR>();
          });
          wait_vmcnt<(ST - 2) * LOADS>();
          barrier_lds();
          sched_fence();
          to_next();
          // NKS is even: the last substep's fragments are in set 1; the
          // loads and tile t+1's first reads go after its MFMAs
          mfmas_then(fa1, fb1, fa0, fb0, std::integral_constant<int, 0>{}, ns, std::integral_constant<int, 0>{},
                     std::integral_constant<int, LOADS>{}, [&](auto part) __attribute__((always_inline)) {
                       issue_tile(cur, prs, qrs, pv, qv, t + ST, cs_, part);
                     });
          sched_interleave<FM * FN, LOADS, DSR>();
        }
      };
      // An even number of tiles (an odd count runs one more tile past the
      // end: its stage holds zeros, which add nothing); with two arrays in
      // pairs, so that each names its stage at compile time.
      if constexpr (TWO) {
        for (int t = 0; t < cur.nk; t += 2) {
          tile(t, lds0, lds1, (uint32_t)STG);
          tile(t + 1, lds1, lds0, (uint32_t)-STG);
        }
      } else {
        const int nk_run = (cur.nk + 1) & ~1;
        for (int t = 0; t < nk_run; ++t) {
          const bool odd = t & 1;
          tile(t, odd ? lds1 : lds0, odd ? lds0 : lds1, odd ? (uint32_t)-STG : (uint32_t)STG);
        }
      }
    }
    // Drain this wave's loads of the tiles past the end (they write LDS).
    wait_vmcnt<0>();
    if constexpr (PAIR) epi = cur.second ? g2.epi : epi_first;

    // 16x16 form with an epilogue input: the input's first 16-row block is
    // requested now, ahead of the next item's loads, so that waiting for it
    // does not wait for them (vector-memory operations complete in order);
    // each later block is requested before the current block's arithmetic
    // and stores (see the epilogue), into the fragment registers the K loop
    // has released. The epilogue's loads and stores are buffer operations
    // without branches: rows past the matrix lie beyond the buffer
    // resource (which starts at the tile's first row), chunks past the last
    // column take kOobOffset. Branches around them would leave the compiler
    // unable to count the operations in flight, and every wait for a block
    // would then wait for the previous block's stores as well.
    constexpr int E_CPR = Cfg::WTN / 8, E_HB = 16, E_PASSES = (E_HB * E_CPR + 63) / 64;
    constexpr bool E_PART = E_PASSES * 64 != E_HB * E_CPR;
    u32x4 zin[M16 && Epi::kInput ? E_PASSES : 1];
    // byte offset of 16-byte chunk c8 of row `row` (both relative to the
    // wave's tile) in a tensor of the epilogue's pitch, rows from the tile's
    // first on; kOobOffset past the last column
    auto e_off = [&](const Item& it, int row, int c8) __attribute__((always_inline)) {
      const int64_t n = it.n0 + wn * Cfg::WTN + c8 * 8;
      return n < sh.N ? (uint32_t)(((int64_t)(wm * Cfg::WTM + row) * epi.ld + n) * 2) : kOobOffset;
    };
    auto e_rsrc = [&](const Item& it, const void* t) __attribute__((always_inline)) {
      return uniform_rsrc(t ? static_cast<const char*>(t) + it.m0 * epi.ld * 2 : nullptr,
                          t ? (sh.M - it.m0) * epi.ld * 2 : 0);
    };
    auto load_input = [&](const Item& it, int rb) __attribute__((always_inline)) {  // rows rb .. rb + 15
      if constexpr (M16 && Epi::kInput) {
        const __amdgpu_buffer_rsrc_t rs = e_rsrc(it, epi.input());
        auto go = [&](auto aux) __attribute__((always_inline)) {
          static_for<0, E_PASSES>([&](auto p) {
            const int q = lane + 64 * p, row = q / E_CPR, c8 = q % E_CPR;
            if (E_PART && p == E_PASSES - 1 && q >= E_HB * E_CPR) return;
            zin[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, e_off(it, rb + row, c8), 0, decltype(aux)::value);
          });
        };
        if (epi.stream) go(std::integral_constant<int, 2>{});  // non-temporal
        else go(std::integral_constant<int, 0>{});
      }
    };
    load_input(cur, 0);
    // The per-column parameters of the wave's columns (the bias), the same
    // for every fragment row: requested here too, branch-free (past the
    // last column: kOobOffset, a zero).
    float colp[Epi::kColParam ? FN : 1];
    if constexpr (Epi::kColParam) {
      const __amdgpu_buffer_rsrc_t crs = uniform_rsrc(epi.colvec(), sh.N * 2);
      static_for<0, FN>([&](auto j) {
        const int64_t n = cur.n0 + wn * Cfg::WTN + j * Cfg::FRAG + (lane & (Cfg::FRAG - 1));
        const uint16_t u = __builtin_amdgcn_raw_buffer_load_b16(crs, n < sh.N ? (uint32_t)(n * 2) : kOobOffset, 0, 0);
        colp[j] = S::to_f((typename S::T)u);
      });
    }

    // Stages: the loop ran an even number of tiles, so the next item's
    // k-tile 0 goes to stage 0 (free: its last reader, of a tile past the
    // end whose data nothing uses, may still be reading; this wave's own
    // loads into it have drained) and the epilogue stages its output
    // through stage 1, which the next item's k-tile 1 will use.
    const int v_next = v + (int)gridDim.x;
    const bool has_next = v_next < nwork;
    if constexpr ((M16 && Epi::kInput) || Epi::kColParam) {
      // Without a branch (so that the compiler counts these loads when it
      // waits for the data requested above): past the last item,
      // empty buffer resources make them fill stage 0 with zeros that
      // nothing reads, and the loads drain before the workgroup ends.
      const Item nxt = decode(opaque_s(has_next ? v_next : v));
      uint32_t pv2[NPV], qv2[NQV];
      offsets(nxt, pv2, qv2);
      const __amdgpu_buffer_rsrc_t none = uniform_rsrc(nullptr, 0);
      const __amdgpu_buffer_rsrc_t prs2 = has_next ? p_rsrc(nxt) : none, qrs2 = has_next ? q_rsrc(nxt) : none;
      issue_tile(nxt, prs2, qrs2, pv2, qv2, 0, lds0, kAll);
    } else if (has_next) {
      const Item nxt = decode(opaque_s(v_next));
      uint32_t pv2[NPV], qv2[NQV];
      offsets(nxt, pv2, qv2);
      const __amdgpu_buffer_rsrc_t prs2 = p_rsrc(nxt), qrs2 = q_rsrc(nxt);
      issue_tile(nxt, prs2, qrs2, pv2, qv2, 0, lds0, kAll);
    }

    const Item done = decode(opaque_s(v));
    const int64_t m0 = done.m0, n0 = done.n0;
    if constexpr (Epi::kDirectF32) {
      // fp32 read-modify-write straight from the accumulators: lanes 0-31
      // and 32-63 each cover 32 consecutive columns (128 bytes) of one row.
      // All 16 loads of a fragment are issued before its stores (written
      // out so: the compiler cannot tell the addresses apart and would
      // otherwise wait for each load in turn).
      static_for<0, FM>([&](auto i) {
        static_for<0, FN>([&](auto j) {
          const int64_t n = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
          const int64_t mf = m0 + wm * Cfg::WTM + i * 32 + 4 * (lane >> 5);
          float* const base = epi.main + mf * epi.ld + n;
          float old[16];
          static_for<0, 16>([&](auto r) {
            const int64_t m = mf + 8 * (r / 4) + (r % 4);
            old[(int)r] = (m < sh.M && n < sh.N) ? base[(8 * (r / 4) + (r % 4)) * epi.ld] : 0.0f;
          });
          static_for<0, 16>([&](auto r) {
            const int64_t m = mf + 8 * (r / 4) + (r % 4);
            if (m < sh.M && n < sh.N) base[(8 * (r / 4) + (r % 4)) * epi.ld] = old[(int)r] + acc[i][j][(int)r];
          });
        });
      });
    } else if (done.part >= 0) {
      // One k-range of a tail tile: the raw fp32 partial sums, in place of
      // the epilogue (tail_finish_kernel applies it).
      float* pt = tail.partial + ((int64_t)(done.tile - tail.full) * tail.parts + done.part) * (BM * BN);
      if constexpr (M16) {
        // lane l holds C[4 (l / 16) + r][l % 16] of each 16x16 fragment
        static_for<0, FM>([&](auto i) {
          static_for<0, FN>([&](auto j) {
            const int c = wn * Cfg::WTN + j * 16 + (lane & 15);
            static_for<0, 4>([&](auto r) {
              const int row = wm * Cfg::WTM + i * 16 + 4 * (lane >> 4) + r;
              pt[row * BN + c] = acc[i][j][(int)r];
            });
          });
        });
      } else static_for<0, FM>([&](auto i) {
        static_for<0, FN>([&](auto j) {
          const int c = wn * Cfg::WTN + j * 32 + (lane & 31);
          static_for<0, 16>([&](auto r) {
            const int row = wm * Cfg::WTM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
            pt[row * BN + c] = acc[i][j][(int)r];
          });
        });
      });
    } else if constexpr (M16) {
      // The 16x16 form's epilogue: per fragment row of the wave's tile (16
      // rows) through a private block of stage 1, as below: the input
      // (if any, requested one block ahead) lands there as 16-byte row
      // chunks and comes back per lane with one transposing read per
      // fragment (lane l holds
      // C[4 (l / 16) + r][l % 16], r = 0..3, of each fragment: four rows of
      // a column); each output is rounded into the block, read back as
      // 16-byte row chunks and stored non-temporally. A second output reuses
      // the block once the first is stored, its fp32 values held in the
      // accumulators meanwhile.
      barrier_lds();
      char* const epi_lds = lds1;
      constexpr int CPR = Cfg::WTN / 8;      // 16-byte chunks per staged row
      constexpr int RS = Cfg::WTN * 2 + 16;  // staged row stride (bytes)
      constexpr int HB = 16, BLK = HB * RS;
      constexpr int PASSES = (HB * CPR + 63) / 64;
      constexpr bool PART = PASSES * 64 != HB * CPR;
      static_assert(Cfg::WAVES * BLK <= STG, "staging fits in one stage");
      char* const stg = epi_lds + wave * BLK;
      const int64_t mw = m0 + wm * Cfg::WTM, nw = n0 + wn * Cfg::WTN;
      const int G = lane >> 4, jj = lane & 15;
      auto store_block = [&](typename S::T* out, int i) __attribute__((always_inline)) {  // fragment row i
        const __amdgpu_buffer_rsrc_t rs = e_rsrc(done, out);
        static_for<0, PASSES>([&](auto p) {
          const int q = lane + 64 * p, row = q / CPR, c8 = q % CPR;
          if (PART && p == PASSES - 1 && q >= HB * CPR) return;
          const u32x4 x = *reinterpret_cast<const u32x4*>(stg + row * RS + c8 * 16);
          __builtin_amdgcn_raw_buffer_store_b128(x, rs, e_off(done, 16 * i + row, c8), 0, 2);  // non-temporal
        });
      };
      float cs[FN];
      static_for<0, FN>([&](auto j) { cs[j] = 0.0f; });
      static_for<0, FM>([&](auto i) {
        const int64_t mb = mw + i * 16;
        if constexpr (Epi::kInput) {
          static_assert(E_PASSES == PASSES && E_CPR == CPR && E_HB == HB, "one block layout");
          static_for<0, PASSES>([&](auto p) {
            const int q = lane + 64 * p, row = q / CPR, c8 = q % CPR;
            if (PART && p == PASSES - 1 && q >= HB * CPR) return;
            *reinterpret_cast<u32x4*>(stg + row * RS + c8 * 16) = zin[p];
          });
          if constexpr (i + 1 < FM) load_input(done, 16 * (i + 1));
        }
        static_for<0, FN>([&](auto j) {
          const int64_t n = nw + j * 16 + jj;
          const bool n_ok = n < sh.N;
          float in[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (Epi::kInput) {
            // rows 4 G + r of column j * 16 + jj: four 16-bit reads (a
            // transposing read here made the compiler wait for every
            // direct-to-LDS load in flight first, the next item's included)
            const char* const pz = stg + 4 * G * RS + (j * 16 + jj) * 2;
#pragma unroll
            for (int r = 0; r < 4; ++r) in[r] = S::to_f(*reinterpret_cast<const typename S::T*>(pz + r * RS));
          }
          static_for<0, 4>([&](auto r) {
            float o[2];
            const float c = epi.eval(acc[i][j][(int)r], Epi::kColParam ? colp[Epi::kColParam ? (int)j : 0] : 0.0f,
                                     in[(int)r], o);
            if constexpr (Epi::kColSum) {
              if (n_ok && mb + 4 * G + r < sh.M) cs[j] += c;
            }
            *reinterpret_cast<typename S::T*>(stg + (4 * G + r) * RS + (j * 16 + jj) * 2) = S::from_f(o[0]);
            if constexpr (Epi::kOuts == 2) acc[i][j][(int)r] = o[1];
          });
        });
        store_block(epi.output(0), i);  // a null output: an empty resource, every store dropped
        if constexpr (Epi::kOuts == 2) {
          if (epi.output(1)) {
            static_for<0, FN>([&](auto j) {
              static_for<0, 4>([&](auto r) {
                *reinterpret_cast<typename S::T*>(stg + (4 * G + r) * RS + (j * 16 + jj) * 2) =
                    S::from_f(acc[i][j][(int)r]);
              });
            });
            store_block(epi.output(1), i);
          }
        }
      });
      if constexpr (Epi::kColSum) {
        // Column sums of this tile, in a fixed order: the four lane groups
        // (pairwise), then the waves along M. LDS-only barriers: the
        // outputs' stores may still be in flight.
        barrier_lds();
        float* red = reinterpret_cast<float*>(epi_lds);  // [WAVES_M][BN]
        static_for<0, FN>([&](auto j) {
          cs[j] += __shfl_xor(cs[j], 16);
          cs[j] += __shfl_xor(cs[j], 32);
        });
        if (lane < 16) static_for<0, FN>([&](auto j) { red[wm * BN + wn * Cfg::WTN + j * 16 + lane] = cs[j]; });
        barrier_lds();
        for (int c = tid; c < BN; c += Cfg::THREADS) {
          float sum = 0.0f;
#pragma unroll
          for (int w = 0; w < Cfg::WAVES_M; ++w) sum += red[w * BN + c];
          if (n0 + c < sh.N) epi.colsum(done.tm, n0 + c, sum);
        }
      }
    } else {
      // Epilogue, one block of 32, 16 or 8 rows of the wave's tile at a
      // time, staged through a private region of stage 1 so that global
      // memory sees whole 16-byte row chunks. The outputs are written with
      // non-temporal stores: no later access of this launch reads them, and
      // when every workgroup finishes a tile at once a burst of ordinary
      // stores displaces operand lines the next items read (measured on
      // MI355X, 16384 x 10240 x 10240 repeated alone: 2.48 -> 2.41 ms for a
      // plain store, 2.62 -> 2.54 ms with the bias + GeLU pair; inside the
      // h=10240 shard's step, whose operands mostly come from HBM anyway,
      // 0.5 % of the step; a one-wave 8192 x 2560 x 2560 launch is
      // unchanged). The input is read the same way when the epilogue says so
      // (epi.stream: an input at least as large as the MALL).
      //
      //   input (if any): 16-byte row chunks -> LDS -> per lane the
      //                   fragment's values via ds_read_b64_tr_b16 (four
      //                   rows of a column);
      //   outputs:        fp32 -> 16-bit, written to LDS at (row, column),
      //                   read back as 16-byte row chunks and stored.
      // Lane l holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] of each 32x32
      // fragment, r = 0..15. The barrier first makes sure no wave still
      // reads fragments of that stage.
      barrier_lds();
      char* const epi_lds = lds1;
      constexpr int CPR = Cfg::WTN / 8;      // 16-byte chunks per staged row
      constexpr int RS = Cfg::WTN * 2 + 16;  // staged row stride (bytes)
      // Rows per staged block: as many (32, 16 or 8) as fit in one stage.
      constexpr int HB = Cfg::WAVES * Epi::kOuts * 32 * RS <= STG   ? 32
                         : Cfg::WAVES * Epi::kOuts * 16 * RS <= STG ? 16
                                                                    : 8;
      constexpr int BLK = HB * RS;                    // one staged block
      constexpr int PASSES = (HB * CPR + 63) / 64;    // chunks per lane per block (the last pass may be partial)
      constexpr bool PART = PASSES * 64 != HB * CPR;
      static_assert(Cfg::WAVES * Epi::kOuts * BLK <= STG, "staging fits in one stage");
      char* const stg = epi_lds + wave * (Epi::kOuts * BLK);
      const int64_t mw = m0 + wm * Cfg::WTM, nw = n0 + wn * Cfg::WTN;
      const int G = lane >> 4, jj = lane & 15;
      float cs[FN];
      static_for<0, FN>([&](auto j) { cs[j] = 0.0f; });
      static_for<0, FM * (32 / HB)>([&](auto ib) {
        constexpr int i = ib / (32 / HB);                // fragment row
        constexpr int g0 = (ib % (32 / HB)) * (HB / 8);  // first 8-row group of the block
        const int64_t mb = mw + i * 32 + g0 * 8;
        if constexpr (Epi::kInput) {
          static_for<0, PASSES>([&](auto p) {
            const int q = lane + 64 * p, row = q / CPR, c8 = q % CPR;
            if (PART && p == PASSES - 1 && q >= HB * CPR) return;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (mb + row < sh.M && nw + c8 * 8 < sh.N) {
              const u32x4* src = reinterpret_cast<const u32x4*>(epi.input() + (mb + row) * epi.ld + nw + c8 * 8);
              x = epi.stream ? __builtin_nontemporal_load(src) : *src;
            }
            *reinterpret_cast<u32x4*>(stg + row * RS + c8 * 16) = x;
          });
        }
        static_for<0, FN>([&](auto j) {
          const int64_t n = nw + j * 32 + (lane & 31);
          const bool n_ok = n < sh.N;
          static_for<0, HB / 8>([&](auto g) {
            float in[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (Epi::kInput) {
              typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
              const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4*)(stg + (8 * g + 4 * (G >> 1) + (jj >> 2)) * RS + ((G & 1) * 16 + (jj & 3) * 4) * 2 +
                               j * 64));
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) in[rr] = S::to_f((typename S::T)(uint16_t)x[rr]);
            }
            static_for<0, 4>([&](auto rr) {
              const int row = 8 * g + 4 * (lane >> 5) + rr;  // within the block
              float o[2];
              const float c = epi.eval(acc[i][j][4 * (g0 + g) + rr],
                                       Epi::kColParam ? colp[Epi::kColParam ? (int)j : 0] : 0.0f, in[rr], o);
              if (n_ok && mb + row < sh.M) cs[j] += c;
              static_for<0, Epi::kOuts>([&](auto k) {
                *reinterpret_cast<typename S::T*>(stg + k * BLK + row * RS + (j * 32 + (lane & 31)) * 2) =
                    S::from_f(o[k]);
              });
            });
          });
        });
        static_for<0, Epi::kOuts>([&](auto k) {
          typename S::T* const out = epi.output(k);
          if (out) {
            static_for<0, PASSES>([&](auto p) {
              const int q = lane + 64 * p, row = q / CPR, c8 = q % CPR;
              if (PART && p == PASSES - 1 && q >= HB * CPR) return;
              const u32x4 x = *reinterpret_cast<const u32x4*>(stg + k * BLK + row * RS + c8 * 16);
              if (mb + row < sh.M && nw + c8 * 8 < sh.N)
                __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(out + (mb + row) * epi.ld + nw + c8 * 8));
            });
          }
        });
      });
      if constexpr (Epi::kColSum) {
        // Column sums of this tile, in a fixed order: the two lane halves,
        // then the waves along M.
        __syncthreads();
        float* red = reinterpret_cast<float*>(epi_lds);  // [WAVES_M][BN]
        static_for<0, FN>([&](auto j) { cs[j] += __shfl_xor(cs[j], 32); });
        if (lane < 32) static_for<0, FN>([&](auto j) { red[wm * BN + wn * Cfg::WTN + j * 32 + lane] = cs[j]; });
        __syncthreads();
        for (int c = tid; c < BN; c += Cfg::THREADS) {
          float sum = 0.0f;
#pragma unroll
          for (int w = 0; w < Cfg::WAVES_M; ++w) sum += red[w * BN + c];
          if (n0 + c < sh.N) epi.colsum(done.tm, n0 + c, sum);
        }
      }
    }
    if (!has_next) {
      if constexpr ((M16 && Epi::kInput) || Epi::kColParam) wait_vmcnt<0>();  // the loads into stage 0 above
      break;
    }
    // Every wave is done with stage s_epi before the next item loads it.
    barrier_lds();
    v = v_next;
  }
}

// Epilogue of the tail tiles of a split launch: C = round(sum of the
// parts' fp32 partials, in part order). One thread per 8 consecutive
// columns of one row of one tail tile.
template <class S, int GROUP, int BM, int BN>
__global__ __launch_bounds__(256) void tail_finish_kernel(const float* partial, int full, int ntail, int parts,
                                                          int tiles_m, int tiles_n, int64_t M, int64_t N,
                                                          typename S::T* out, int64_t ld) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (tail tile, row, 8-column chunk)
  constexpr int CH = BN / 8;
  const int64_t per_tile = (int64_t)BM * CH;
  const int q = (int)(idx / per_tile);
  if (q >= ntail) return;
  const int rem = (int)(idx % per_tile), row = rem / CH, c8 = rem % CH;
  int tm, tn;
  tile_coords<GROUP>(full + q, tiles_m, tiles_n, tm, tn);
  const int64_t m = (int64_t)tm * BM + row, n = (int64_t)tn * BN + c8 * 8;
  if (m >= M || n >= N) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < parts; ++p) {
    const float* src = partial + ((int64_t)q * parts + p) * (BM * BN) + row * BN + c8 * 8;
    const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += a[e];
      acc[4 + e] += b[e];
    }
  }
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    v[e] = (uint32_t)S::from_f(acc[2 * e]) | ((uint32_t)S::from_f(acc[2 * e + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + m * ld + n) = v;
}

}  // namespace tpmlp
