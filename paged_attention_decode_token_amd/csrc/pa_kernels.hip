// Paged-attention decode kernels for gfx950 (MI355X).
//
// Tile kernel: one workgroup per task (sequence b, KV head, partition = a
// contiguous range of 256-token tiles; ROCm/aiter PR #7092, "Root cause").
// Four waves split every tile into 64-token slices and keep a wave-private
// online softmax (running max m, weight sum l, accumulator O) over their
// slices, with no barrier in the tile loop; the four waves merge once at the
// end (ROCm/aiter PR #7056, "Behavior and intent").
//
// Per 64-token slice and wave:
//   QK  S^T[token][row] = K . Q^T on v_mfma_f32_16x16x32_bf16 (bf16 cache; an
//       e4m3 cache is widened to bf16 exactly), or on the block-scaled
//       v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 K (e8m0 scale per 32) and
//       e4m3 Q for an MXFP4 cache (PR #7056, "Summary").
//   softmax in base 2, row max across the wave with cross-lane shuffles.
//   PV  O^T[d][row] += V^T . P^T on the bf16 MFMA, P rounded to bf16. Token-
//       major V goes through a wave-private LDS tile and is read back
//       transposed with ds_read_b64_tr_b16; a transposed V feeds the MFMA
//       straight from its loads.
// Only the last, partial tile of a sequence runs the masked variant
// (PR #7092, "Fix"): scores of tokens >= L become -inf by a select, and V
// bytes and per-token scales of those tokens are zeroed before the PV
// product, so 0 * NaN can never reach the accumulator. Tiles past
// ceil(L/256) and table columns past ceil(L/page) are never read; page slots
// of the boundary tile beyond the last owned page read block 0 and are
// masked like any other unowned row.
//
// Merge kernel: per output row, combines the partitions' (m, l, O) with a
// log-sum-exp weighting in a fixed partition order and writes bf16.
//
// Lane layouts of the matrix instructions used here (measured on gfx950):
//   16x16x32 bf16: A lane (m, g) holds A[m][8g..8g+7], B lane (n, g) holds
//     B[8g..8g+7][n], C lane (n, g) holds C[4g..4g+3][n]  (m, n = lane % 16,
//     g = lane / 16).
//   16x16x128 f8f6f4 with fp4 A: A lane (m, g) nibble i (element 2i in the
//     low nibble) is k = 32g + i; an fp8 B lane (n, g) byte j is
//     k = 16g + j for j < 16 and k = 64 + 16g + (j - 16) for j >= 16; the
//     scale byte of lane group g applies to k in [32g, 32g + 32) on both
//     operands (the placement PR #7056 describes for its fold).
//   ds_read_b64_tr_b16: within each 16-lane group, output lane i element e
//     comes from source lane 4e + i/4, element i % 4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define PA_DEV __device__ __forceinline__

// Online softmax: how far (base 2) a row's max may grow past the reference
// max before the weights are re-based and O rescaled. Weights stay below
// 2^kRescaleLog2 = 256, well inside bf16 and fp32 range.
constexpr float kRescaleLog2 = 8.f;

// ------------------------------------------------------------------ helpers

PA_DEV u32x4 ld16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
PA_DEV u32x2 ld8(const char* p) { return *reinterpret_cast<const u32x2*>(p); }
PA_DEV uint32_t ld4(const char* p) { return *reinterpret_cast<const uint32_t*>(p); }
// KV cache bytes are read once per call. Nontemporal loads stream faster on
// gfx950 (about 6.9 against 6.2 TB/s for 16 KB pages read 1 KB per
// instruction), but only when each instruction covers whole 128-byte lines:
// where one instruction reads half of a line and a later one (or another
// wave) the other half, the evict-first line is fetched again and the rate
// drops below that of ordinary loads (5.6 TB/s for the 16-rows x 64-byte
// pattern of an MFMA A operand). So they are used for token-major V staging
// (a lane group reads whole rows) and for MXFP4 K (64-byte rows, four adjacent
// tokens per instruction), and not for K rows of 128 bytes or more, transposed
// V rows split between two waves, or per-token scales shared between heads.
PA_DEV u32x4 ld16_kv(const char* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
constexpr int kLoadNontemporal = 2;  // cache-policy operand of the LDS DMA load: nt
PA_DEV uint32_t ld4_kv(const char* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }

PA_DEV int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// s_waitcnt immediate that waits until at most n vector-memory instructions
// are outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

PA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

PA_DEV float shfl_xor(float v, int mask) {
    int lane = __lane_id();
    int src = lane ^ mask;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

PA_DEV uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
PA_DEV float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
PA_DEV float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two e4m3 bytes (selected 16-bit half of w) -> two bf16 (exact: every e4m3
// value is a bf16 value).
template <bool HI>
PA_DEV uint32_t fp8x2_to_bf16x2(uint32_t w) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}
// Four e4m3 bytes -> four bf16 in two dwords.
PA_DEV u32x2 fp8x4_to_bf16x4(uint32_t w) {
    u32x2 r;
    r[0] = fp8x2_to_bf16x2<false>(w);
    r[1] = fp8x2_to_bf16x2<true>(w);
    return r;
}
// Eight e4m3 bytes -> bf16x8 fragment.
PA_DEV bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    u32x2 a = fp8x4_to_bf16x4(w0), b = fp8x4_to_bf16x4(w1);
    u32x4 r = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, r);
}

// e8m0 byte -> fp32 2^(byte - 127) (byte 0 gives the subnormal 2^-127).
PA_DEV float e8m0_to_f32(uint32_t byte) {
    return byte == 0 ? __builtin_bit_cast(float, 0x00400000u) : __builtin_bit_cast(float, byte << 23);
}

// Eight e2m1 values (one dword, element 2i in the low nibble of byte i) times
// `scale` -> bf16x8 (exact for the scales an e8m0 byte in [1, 254] encodes
// times any e2m1 value).
template <int SEL>
PA_DEV uint32_t fp4x2_to_bf16x2(uint32_t w, float scale) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL);
    return __builtin_bit_cast(uint32_t, r);
}
PA_DEV u32x4 fp4x8_to_bf16x8(uint32_t w, float scale) {
    u32x4 r;
    r[0] = fp4x2_to_bf16x2<0>(w, scale);
    r[1] = fp4x2_to_bf16x2<1>(w, scale);
    r[2] = fp4x2_to_bf16x2<2>(w, scale);
    r[3] = fp4x2_to_bf16x2<3>(w, scale);
    return r;
}

PA_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

PA_DEV f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Byte mask keeping the first `valid` bytes (valid clamped to 0..4) of a dword.
PA_DEV uint32_t keep_bytes(int valid) {
    valid = valid < 0 ? 0 : (valid > 4 ? 4 : valid);
    return valid >= 4 ? 0xFFFFFFFFu : ((1u << (8 * valid)) - 1u);
}

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// ----------------------------------------------------------- configuration

template <int KV_, int SC_, int VT_, int D_, int PG_, int NT_, int QF8_, int MXS_, int WIN_>
struct Cfg {
    // WIN_ 1: a sliding window (with or without causal rows): masked tiles may
    // open the range (the window's first tiles, with the rows before the
    // window inert) and close it before the context boundary. WIN_ 2: causal
    // rows without a window: each row ends at its own position, at most
    // qlen - 1 tokens before L, so every score gets a select against the row's
    // end (no V byte past it is unowned), and only the last tile runs masked.
    static constexpr bool WIN = WIN_ == 1;
    static constexpr bool ROWS = WIN_ != 0;    // per-row range ends
    static constexpr bool CAUSAL = WIN_ == 2;  // the select in unmasked tiles
    static constexpr int KV = KV_;
    static constexpr int SC = SC_;
    static constexpr bool VT = VT_ != 0;
    static constexpr int D = D_;
    static constexpr int PG = PG_;
    static constexpr int NT = NT_;  // 16-row N tiles of query rows (rows <= 16 * NT)
    static constexpr bool QF8 = QF8_ != 0;
    // MXFP4 QK on the block-scaled fp4 x fp8 MFMA (opt-in) instead of exact
    // widening of K to bf16 and the bf16 MFMA (default). On gfx950 the scaled
    // instruction keeps one 32-element block's sum to about 2^-14 of the
    // block's largest product (2^-12.6 with the query scaled up to 448),
    // however the 128-deep reduction is split across instructions; near-tied
    // logits can turn that into output errors above the element bound. The
    // widened form is exact up to fp32 accumulation.
    static constexpr bool MXS = KV_ == KV_MXFP4 && MXS_ != 0;
    // P enters PV as bf16 hi + lo parts (two MFMAs) for MXFP4: its softmax is
    // near one-hot and its V rows reach 6 * 2^9, so bf16 rounding of a
    // runner-up weight alone would move an output element by far more than the
    // element bound wherever the mixed V rows cancel. Also with per-token V
    // scales: the weight P * v_scale has no exact bf16 form and the weight
    // sum cannot share its rounding, so one bf16 rounding adds about 2^-9 / 3
    // of relative error per weight on top of the bf16 output rounding (rel-L2
    // 2.95e-3 against a 2.30e-3 output-rounding floor on 64 rows of a mixed
    // short-length batch); hi + lo leaves only the output rounding. Only with
    // 64 query rows: at 16 and 32 rows the second P*V product costs time (1 us
    // of a 63 us tile kernel at 16 rows) or registers (the head_dim-256 loop
    // spills at 32 rows), and one rounding gives rel-L2 2.4e-3 on the fp8
    // per-token batch against a 1.7e-3 floor.
    static constexpr bool PSPLIT = KV == KV_MXFP4 || (SC_ == SC_TOKEN && NT_ == 4);
    static constexpr int ESZ = KV == KV_BF16 ? 2 : 1;                // bytes per bf16/fp8 element
    static constexpr int ROWB = KV == KV_MXFP4 ? D / 2 : D * ESZ;    // bytes of one token row (data)
    static constexpr int SROWB = KV == KV_MXFP4 ? D / 32 : 0;        // bytes of one token's e8m0 scales
    static constexpr int KSTEPS = D / 32;                            // bf16 MFMA k-steps per 16 tokens
    static constexpr int KLOADS = KV == KV_MXFP4 ? 1 : ROWB / 64;    // 16-byte K loads per lane per call
    static constexpr int DT = D / 16;                                // 16-wide d tiles of O
    static constexpr int NPC = PG >= 64 ? 1 : 64 / PG;               // pages per 64-token slice
    static constexpr long PAGE_BYTES_HEAD = (long)PG * ROWB;         // one (page, head) of K or V data
    // Token-major V of a bf16 or e4m3 cache goes straight from HBM into a
    // wave-private LDS tile (64 token rows, XOR-swizzled 16-byte chunks) by
    // LDS DMA and is read back transposed; MXFP4 V is widened to bf16 in
    // registers and staged through LDS one 32-token PV step at a time.
    // Measured per configuration: one N tile (32 query rows only in the fp8
    // per-token case below), and not for bf16 pages of 64 or 128 tokens without
    // a window (there the register path at one workgroup per CU beats the DMA
    // path at one or two on the batch-64 workload: 179.5 against 183-209 us at
    // page 128, 174 against 184 us at page 64). The windowed bf16 page-64
    // instance keeps the DMA path (window 1024: 51.8 against 55.2 us).
    //
    // The wait before PV allows the KVMEM loads issued after the slice's DMA to
    // be outstanding. Loads, the DMA included, complete in issue order, and any
    // other memory operation issued after the DMA (a spill) only adds to the
    // outstanding count, so the wait stays sufficient with spills; they cost
    // time, not correctness.
    //
    // fp8 per-token caches with 32 query rows at head_dim 256 take the DMA path
    // (with the query fragments in LDS, which keeps the loop free of spills)
    // wherever the register-staged loop spills to scratch: in the windowed
    // instances and at page 64, where each scratch reload in the loop waits for
    // every load in flight (qlen 4, batch 16: 82-87 against 90-118 us per call).
    // The plain page-16 and page-128 instances keep register staging, whose
    // loops do not spill and which measured faster there (80-81 against 99 us).
    static constexpr bool NT2_DMA = KV_ == KV_FP8 && SC_ == SC_TOKEN && NT_ == 2 && D_ == 256 && (WIN_ == 1 || PG_ == 64);
    // 64 query rows (four N tiles, head_dim 128 only): the accumulators alone
    // take 128 registers, so V always goes by LDS DMA and the query fragments
    // live in LDS, leaving the registers to K, the scores and O.
    static constexpr bool NT4 = NT_ == 4;
    static constexpr bool VDMA = !VT && KV != KV_MXFP4 && (NT_ == 1 || NT2_DMA || NT4) &&
                                 !(KV_ == KV_BF16 && !NT4 && (PG_ == 128 || (PG_ == 64 && WIN_ == 0)));
    static constexpr bool STAGE_V = !VT && !VDMA;
    // Register-staged V loads held at the top of the slice (see load_v): for
    // the fp8 per-token page-16 instance with 32 query rows at head_dim 256,
    // where it also removes every spill (qlen 4, batch 16: 80.7 -> 76.2 us per
    // call); at page 128 it adds a spill reload to the loop (80.1 -> 86.9 us).
    static constexpr bool PIN_V = STAGE_V && KV_ == KV_FP8 && SC_ == SC_TOKEN && NT_ == 2 && D_ == 256 && PG_ == 16;
    // Whole-stage prefetch (fp8 caches with per-token scales on the LDS-DMA
    // path, one workgroup per CU): the K, V and scale loads of a wave's next
    // slice are all issued at the top of the current one, into a second K
    // register set, a second V tile and a second scale block (the scales also
    // arrive by LDS DMA). One full wait per slice then covers exactly the
    // slice about to be computed, so a slice costs max(load latency, compute)
    // rather than their sum: with K in one register set, the next slice's K
    // can only be issued after this slice's QK has read it. (The compiler waits
    // for everything outstanding before using a register loaded ahead of an
    // LDS DMA, so register loads cannot be kept in flight across a DMA wait;
    // hence the one full wait at the top.)
    static constexpr bool PF = VDMA && KV_ == KV_FP8 && SC_ == SC_TOKEN && NT_ == 1;
    // Lazy softmax rescaling (qk_softmax) in the whole-stage-prefetch
    // instances, where it measured faster (fp8 per-token qlen 1: 71.0 -> 70.3
    // us per call). With more than one N tile the register allocation around
    // its branch spills in the loops of the head_dim-256 and 64-row
    // instances; in the other one-tile instances it measured no faster, and
    // at bf16 page 128 its smaller register count lets a second workgroup in,
    // which is slower there.
    static constexpr bool LAZY = PF;
    // Whole-line K loads (load_k, fix_k) at head_dim 128 with one N tile, in
    // the bf16 instances and the fp8 per-tensor transposed-V ones (with
    // per-token scales those already spill at three workgroups per CU, and
    // whole-line K adds to it): each load instruction
    // reads whole 128-byte lines of 8 tokens, nontemporally, and one lane
    // exchange per register then restores the MFMA operand layout. Measured
    // cold per call, us: bf16 batch 64, 171.6 against 174.1 at page 64 and
    // 177.7 against 180.0 at page 128, 50.2 against 52.0 with a 1024-token
    // window (V by DMA); fp8 transposed V, batch 256 x 16384, 165.0 against
    // 182.6. Not used where it measured no faster: head_dim 256 (bf16, 369
    // against 364 at page 64), the fp8 per-token prefetch instance (70.1
    // against 70.3, qlen 1) and its 32-row instances (75.9 against 76.1 at
    // qlen 4, 68.7 against 68.4 with causal rows).
    static constexpr bool KLINE = NT_ == 1 && D_ == 128 && (KV_ == KV_BF16 || (KV_ == KV_FP8 && VT_ && SC_ != SC_TOKEN));
    // The register-staged bf16 ones are held to one workgroup per compute
    // unit by their LDS reservation (SMEM_ALLOC): at page 64 whole-line K
    // frees the registers for a second one, which measured slower (a split
    // plan and a merge: 180.9 against 174.6 us per call).
    static constexpr bool ONE_PER_CU = KLINE && KV_ == KV_BF16 && STAGE_V;
    static_assert(!(KLINE && PF), "fix_k runs in the loop without the whole-stage prefetch only");
    // query fragments in LDS (one copy per workgroup) instead of registers
    static constexpr bool QLDS = NT2_DMA || NT4;
    // register-staged V tile (bf16 rows): row pitch, extra offset per group of
    // 8 rows, and a gap after every 2^VGSH chunks of a row, in bytes (sv_row, sv_chunk)
    static constexpr int VPITCH = D == 256 ? 544 : KV == KV_BF16 ? 288 : KV == KV_MXFP4 ? 320 : 272;
    static constexpr int VGRP = D == 256 || KV == KV_BF16 ? 128 : KV == KV_MXFP4 ? 32 : 0;
    static constexpr int VGAP = D == 256 || KV == KV_MXFP4 ? 16 : 0;
    static constexpr int VGSH = D == 256 ? 4 : 2;
    static constexpr int CPR = ROWB / 16;                            // 16-byte chunks per V row (DMA)
    static constexpr int VSTAGE_BYTES = VDMA ? 64 * ROWB : (STAGE_V ? 32 * VPITCH + 3 * VGRP : 0);  // per wave
    static constexpr int SCALE_BYTES = PF ? 512 : 0;                 // K then V scales of 64 tokens (fp32)
    static constexpr int WAVE_LDS = (PF ? 2 : 1) * (VSTAGE_BYTES + SCALE_BYTES);  // per wave
    static constexpr int QLDS_BYTES = QLDS ? NT * KSTEPS * 64 * 16 : 0;
    static constexpr int ROWS_PAD = 16 * NT;
    static constexpr int OPITCH = D + 4;                             // floats
    static constexpr int EPI_BYTES = 2 * ROWS_PAD * OPITCH * 4 + 2 * 4 * ROWS_PAD * 4;
    static constexpr int SMEM = (4 * WAVE_LDS + QLDS_BYTES > EPI_BYTES) ? 4 * WAVE_LDS + QLDS_BYTES : EPI_BYTES;
    static constexpr int kLdsPerCu = 160 * 1024;
    static constexpr int SMEM_ALLOC = ONE_PER_CU && SMEM <= kLdsPerCu / 2 ? kLdsPerCu / 2 + 256 : SMEM;
    // staging geometry for token-major V loads
    static constexpr int LPR = ROWB / 16;         // lanes per token row
    static constexpr int TPI = 64 / LPR;          // tokens per load instruction
    static constexpr int IPS = 32 / TPI;          // load instructions per 32-token step
    // Workgroups per compute unit the register allocation is held to. The loop
    // keeps one slice of K or V in flight per wave, so resident waves are what
    // hides HBM latency. These configurations fit 3 (<= 168 VGPRs) or 2
    // (<= 256) waves per SIMD without spilling the loop.
    static constexpr int MINB = (KV == KV_FP8 && VT && D == 128 && NT == 1) || KV == KV_MXFP4 ? 3
                                : (KV == KV_BF16 && VDMA && D == 128 && NT == 1)              ? 2
                                                                                              : 1;
    // vector-memory instructions load_k issues (the explicit wait before PV counts them)
    static constexpr int KVMEM = 4 * KLOADS + (KV == KV_MXFP4 ? 4 : 0) + (SC == SC_TOKEN ? 8 : 0);
};

// Chunk swizzle of the DMA'd V tile: row r (slice token r) stores its 16-byte
// chunk c at position c ^ vswz(r). Chosen so that the 32 lanes of a half-wave
// reading one PV fragment touch 64 distinct LDS banks:
//   bf16 (ds_read_b64_tr_b16): a half-wave reads 32 bytes of rows
//     16g + 8s + [0, 4) (+ 4) for g in {2h, 2h + 1}; the XOR moves bits 1..3
//     of the chunk by (r & 3) and bit 4 of r;
//   e4m3 (ds_read_b64_tr_b8): a half-wave reads 16 bytes of rows
//     16g + 8s + [0, 8); with 256-byte rows the XOR is (r & 7) and bit 4 of r,
//     with 128-byte rows (two rows per 64 banks) it is ((r >> 1) & 3) and bit 4.
template <class C>
PA_DEV int vswz(int r) {
    if constexpr (C::KV == KV_BF16) return 2 * ((r & 3) | (((r >> 4) & 1) << 2));
    else if constexpr (C::ROWB >= 256) return (r & 7) | (((r >> 4) & 1) << 3);
    else return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}

// Layout of the register-staged V tile: bf16 rows of D / 8 chunks of 16
// bytes; row e (= 8 g + token within the step's 8-token half) holds chunk k at
// byte sv_row(e) + sv_chunk(k). The offsets are the lane's base plus constants, and both
// sides avoid LDS bank conflicts (64 banks of 4 bytes):
//   the PV reads (ds_read_b64_tr_b16): a half-wave reads chunks 2dt and
//     2dt + 1 of rows 8g + [0, 4) (+ 4) for g in {2h, 2h + 1}: the row pitch
//     and the per-8-row offset put those 8 rows in 8 different 32-byte bank
//     windows;
//   the staging writes (16 bytes a lane): a 16-lane pass writes chunks c v + j
//     (c = 1, 2 or 4 chunks a lane) of 16 / (D / 8 / c) consecutive rows; the
//     gap inside a row keeps chunks 256 bytes apart (head_dim 256) or a
//     lane's 4 chunks (MXFP4) off each other's banks.
// Conflict-free both ways for bf16 and MXFP4 at head_dim 128 and for head_dim
// 256; fp8 at head_dim 128 keeps 2-way reads (no pitch of this form clears
// both its reads and its writes).
template <class C>
PA_DEV int sv_row(int e) {
    return e * C::VPITCH + (e >> 3) * C::VGRP;
}
template <class C>
PA_DEV int sv_chunk(int k) {
    return 16 * k + C::VGAP * (k >> C::VGSH);
}
// Callers split both terms into the lane's part and a compile-time part: with
// a power-of-two count of rows per load instruction, (i TPI + l) >> 3 =
// ((i TPI) >> 3) + (l >> 3) for l < TPI, and a lane's c chunks (c <= 2^VGSH,
// starting at a multiple of c) never straddle a gap.

template <class C>
struct State {
    f32x4 o[C::DT][C::NT];  // O^T[16dt + 4g + j][16nt + n]
    float m[C::NT];         // running max of the row, base-2 logits
    float l[C::NT];         // running sum of weights (this lane's tokens only)
};

struct Ctx {
    int b, kvh, L, npages, lane, ln, lg, wave;
    // With causal rows or a window: s_lo is the smallest row start of the
    // call. Tokens before it are seen by no row and are treated like tokens
    // at or past L (V bytes and per-token V scales zeroed on masked tiles);
    // table columns before pg_first (= s_lo / page) lie wholly before it and
    // are never read. Without a mask both are 0.
    int s_lo, pg_first;
    int row_s[4], row_e[4];  // token range [row_s, row_e) of this lane's query row in N tile nt
    const int32_t* bt_row;
    const char* kbase;   // K data of this head in page 0
    const char* vbase;   // V data of this head in page 0
    const char* ksbase;  // per-token / MXFP4 scales of this head in page 0
    const char* vsbase;
    float kscale;        // per-tensor K scale (1 otherwise)
};

// Query fragments (B operand of QK).
template <class C>
struct QFrag {
    bf16x8 q[C::NT][C::KSTEPS];  // bf16 B operand (bf16 / fp8 caches, exact MXFP4 QK)
    i32x8 q8[C::NT];             // e4m3 B operand of the scaled MXFP4 QK
    int qsc[C::NT];              // its e8m0 scale byte (2^e of the query row)
};

// d index held at position 0 of the bf16 Q/K fragment for k-step ks, lane group g.
template <class C>
PA_DEV int kfrag_d0(int ks, int g) {
    if (C::KV == KV_BF16)
        return 32 * ks + 8 * g;
    return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1);  // fp8: one 16-byte load feeds two k-steps
}

template <class C>
PA_DEV void load_q(const TileArgs& a, const Ctx& cx, QFrag<C>& qf) {
    const int Hq = a.num_kv_heads * a.q_per_kv;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        const int r = 16 * nt + cx.ln;
        const bool valid = r < a.rows;
        const int rr = valid ? r : 0;
        const long row = ((long)cx.b * a.qlen + rr / a.q_per_kv) * Hq + (long)cx.kvh * a.q_per_kv + rr % a.q_per_kv;
        if constexpr (C::KV != KV_MXFP4) {
            const char* qp = reinterpret_cast<const char*>(a.q) + row * C::D * 2;
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
                u32x4 v = ld16(qp + 2 * kfrag_d0<C>(ks, cx.lg));
                if (!valid) v = u32x4{0, 0, 0, 0};
                qf.q[nt][ks] = as_bf16x8(v);
            }
        } else {
            // MXFP4: this lane's 32 query elements as e4m3 bytes. Scaled QK
            // wants d = 16g + [0,16) then 64 + 16g + [0,16) (the fp8 B layout of
            // the 16x16x128 scaled MFMA); exact QK wants d = 32g + [0,32).
            auto pos = [&](int j) -> int {
                if constexpr (C::MXS) return j < 16 ? 16 * cx.lg + j : 64 + 16 * cx.lg + (j - 16);
                return 32 * cx.lg + j;
            };
            uint32_t bytes[8];
            int e = 0;
            if constexpr (C::QF8) {
                // e4m3 query used as stored, unit scale
                const char* qp = reinterpret_cast<const char*>(a.q) + row * C::D;
                u32x4 lo = ld16(qp + pos(0)), hi = ld16(qp + pos(16));
                if (!valid) { lo = u32x4{0, 0, 0, 0}; hi = lo; }
#pragma unroll
                for (int k = 0; k < 4; ++k) { bytes[k] = lo[k]; bytes[4 + k] = hi[k]; }
            } else {
                // bf16 query row quantized to e4m3 with a power-of-two scale 2^e,
                // e the smallest integer with max|q| <= 448 * 2^e (0 for a zero row)
                const char* qp = reinterpret_cast<const char*>(a.q) + row * C::D * 2;
                float x[32];
                u32x4 w[4] = {ld16(qp + 2 * pos(0)), ld16(qp + 2 * pos(8)), ld16(qp + 2 * pos(16)), ld16(qp + 2 * pos(24))};
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t d = valid ? w[k][j] : 0u;
                        x[8 * k + 2 * j] = bf16_lo(d);
                        x[8 * k + 2 * j + 1] = bf16_hi(d);
                    }
                float amax = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
                amax = fmaxf(amax, shfl_xor(amax, 16));
                amax = fmaxf(amax, shfl_xor(amax, 32));
                if (amax > 0.f) {
                    int ex;
                    float fr = frexpf(amax, &ex);  // amax = fr * 2^ex, fr in [0.5, 1)
                    e = (fr <= 0.875f) ? ex - 9 : ex - 8;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    float f0 = ldexpf(x[4 * k + 0], -e), f1 = ldexpf(x[4 * k + 1], -e);
                    float f2 = ldexpf(x[4 * k + 2], -e), f3 = ldexpf(x[4 * k + 3], -e);
                    int t = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);  // round to nearest even
                    bytes[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, t, true);
                }
            }
            if constexpr (C::MXS) {
                qf.q8[nt] = i32x8{(int)bytes[0], (int)bytes[1], (int)bytes[2], (int)bytes[3],
                                  (int)bytes[4], (int)bytes[5], (int)bytes[6], (int)bytes[7]};
                const int sb = 127 + e;
                qf.qsc[nt] = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
            } else {
                // widen qhat * 2^e to bf16 (exact): k-step s holds d = 32g + 8s + [0, 8)
                const float qs = ldexpf(1.0f, e);
#pragma unroll
                for (int st = 0; st < C::KSTEPS; ++st) {
                    u32x4 v;
                    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)bytes[2 * st], qs, false));
                    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)bytes[2 * st], qs, true));
                    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)bytes[2 * st + 1], qs, false));
                    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)bytes[2 * st + 1], qs, true));
                    qf.q[nt][st] = as_bf16x8(v);
                }
            }
        }
    }
}

// Page id of table slot `slot` (pinned to block 0 past the owned pages and,
// with causal rows or a window, before the first column any row reads;
// clamped into the pool).
template <class C, bool MASK>
PA_DEV int page_of(const TileArgs& a, const Ctx& cx, int slot) {
    // The read is unconditional, since a per-lane branch here would make every
    // loop that refills page ids divergent. Outside the read columns it
    // re-reads the nearest one, and the select pins the slot to block 0. The
    // in-range test is one comparison: with two, the compiler skips the load
    // for the lanes the select discards, which is such a branch.
    int p;
    if constexpr (C::WIN) {
        const int col = MASK ? min(max(slot, cx.pg_first), max(cx.npages - 1, 0)) : slot;
        p = cx.bt_row[col];
        if (MASK && (unsigned)(slot - cx.pg_first) >= (unsigned)(cx.npages - cx.pg_first)) p = 0;
    } else {
        const int col = MASK ? min(slot, max(cx.npages - 1, 0)) : slot;
        p = cx.bt_row[col];
        if (MASK && slot >= cx.npages) p = 0;
    }
    p = p < 0 ? 0 : (p >= a.num_blocks ? a.num_blocks - 1 : p);
    return p;
}

// ------------------------------------------------------ per-slice stages
//
// A wave processes the 64-token slice [cb, cb + 64) of every tile of its task.
// The work is split into load stages (addresses + global loads into
// registers) and compute stages, so that the loads of slice i + 1 are in
// flight while slice i computes: K(i + 1) is issued after QK(i), V(i + 1)
// after PV(i). Loads never depend on whether a slice is the boundary slice;
// page slots past the owned pages read block 0 and the compute stages mask.

template <class C>
struct SlicePages {
    int pg[C::NPC];  // uniform page ids of the slice (compile-time indexed only)
    int kpage;       // page of this lane's K rows
    int tpage;       // page of this lane's 16 score / transposed-V tokens
    int cb;
};

template <class C>
struct KBuf {
    u32x4 k[4][C::KLOADS];  // call c: token 16*(ln>>2) + 4c + (ln&3), bytes 64u + 16*lg
    uint32_t ksc[4];        // MXFP4: the 4 e8m0 bytes of those tokens (byte lg is this lane's block)
    float tks[16], tvs[16]; // per-token scales of tokens 16*lg + [0, 16)
};

template <class C>
struct VBuf {
    u32x4 v[C::STAGE_V ? 2 : 1][C::STAGE_V ? C::IPS : 1];  // token-major rows to stage
    uint32_t vsc[C::STAGE_V ? 2 : 1][C::STAGE_V ? C::IPS : 1];
    u32x4 vt[C::VT ? C::DT : 1][C::VT ? (C::ESZ == 2 ? 2 : 1) : 1];  // transposed V
};

template <class C>
struct PFrag {
    u32x4 hi[2][C::NT];  // P^T B operand of PV steps 0 / 1 (bf16)
    u32x4 lo[2][C::NT];  // low parts when PSPLIT
};

// slot inside its page of slice token t (t in [0, 64))
template <class C>
PA_DEV int slot_in_page(const SlicePages<C>& sp, int t) {
    if constexpr (C::NPC == 1) return (C::PG > 64 ? (sp.cb % C::PG) : 0) + t;
    return t & (C::PG - 1);
}

// Page ids of upcoming slices, prefetched one VGPR at a time so the KV loads
// of a slice never wait on a block-table read: lane l holds the page of slot q
// = l % NPC of the wave's slice in tile `tile0 + l / NPC` (block 0 past the
// owned pages, clamped into the pool).
template <class C>
struct PageCache {
    static constexpr int SPAN = 64 / C::NPC;  // slices covered by one load
    int tile0;
    int pgv;
};

template <class C>
PA_DEV void page_cache_fill(const TileArgs& a, const Ctx& cx, PageCache<C>& pc, int tile0) {
    pc.tile0 = tile0;
    const int tile = tile0 + cx.lane / C::NPC;
    const int slot = (tile * kTileTokens + 64 * cx.wave) / C::PG + cx.lane % C::NPC;
    pc.pgv = page_of<C, true>(a, cx, slot);
    // With pages longer than a slice, a slice that starts at or past L can lie
    // in the last owned page: it reads block 0 as well (the same rows for every
    // task, so mostly from L2) instead of the page's unowned rows from HBM. The
    // last tile's masks discard its scores and zero its V either way.
    if constexpr (C::PG > 64)
        if (tile * kTileTokens + 64 * cx.wave >= cx.L) pc.pgv = 0;
}

PA_DEV int lane_value(int v, int src_lane) { return __builtin_amdgcn_ds_bpermute(src_lane << 2, v); }

template <class C>
PA_DEV SlicePages<C> slice_pages(const TileArgs& a, const Ctx& cx, PageCache<C>& pc, int tile) {
    if (tile - pc.tile0 >= PageCache<C>::SPAN) page_cache_fill(a, cx, pc, tile);
    const int base = (tile - pc.tile0) * C::NPC;
    SlicePages<C> sp;
    sp.cb = tile * kTileTokens + 64 * cx.wave;
#pragma unroll
    for (int q = 0; q < C::NPC; ++q) sp.pg[q] = __builtin_amdgcn_readlane(pc.pgv, base + q);
    if constexpr (C::NPC == 1) {
        sp.kpage = sp.tpage = sp.pg[0];
    } else {
        sp.kpage = lane_value(pc.pgv, base + (cx.ln >> 2));  // token 16*(ln>>2) + ..
        sp.tpage = lane_value(pc.pgv, base + cx.lg);         // token 16*lg + ..
    }
    return sp;
}

template <class C>
PA_DEV void load_k(const TileArgs& a, const Ctx& cx, const SlicePages<C>& sp, KBuf<C>& kb) {
    constexpr int PG = C::PG;
    const int ln = cx.ln, lg = cx.lg;
    const int ktok0 = 16 * (ln >> 2) + (ln & 3);
    if constexpr (C::KLINE) {
        // Lanes ln = 2p and 2p + 1 read the two 64-byte halves of one line:
        // call (c, 2L) line L of token t(2p) = 16*(ln>>2) + (ln&2) + 4c, call
        // (c, 2L + 1) line L of token t(2p) + 1 (same page). Each call then
        // covers line L of 8 whole token rows; fix_k exchanges the halves.
        const char* krow = cx.kbase + (long)sp.kpage * a.num_kv_heads * C::PAGE_BYTES_HEAD +
                           (long)slot_in_page(sp, ktok0 & ~1) * C::ROWB + 64 * (ln & 1) + 16 * lg;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int L = 0; L < C::KLOADS / 2; ++L) {
                const char* src = krow + 4 * c * C::ROWB + 128 * L;
                kb.k[c][2 * L] = ld16_kv(src);
                kb.k[c][2 * L + 1] = ld16_kv(src + C::ROWB);
            }
    } else {
        const char* krow = cx.kbase + (long)sp.kpage * a.num_kv_heads * C::PAGE_BYTES_HEAD +
                           (long)slot_in_page(sp, ktok0) * C::ROWB;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int u = 0; u < C::KLOADS; ++u) {
                const char* src = krow + 4 * c * C::ROWB + 64 * u + 16 * lg;
                kb.k[c][u] = C::ROWB <= 64 ? ld16_kv(src) : ld16(src);
            }
    }
    if constexpr (C::KV == KV_MXFP4) {
        const char* srow = cx.ksbase + (long)sp.kpage * a.num_kv_heads * PG * C::SROWB +
                           (long)slot_in_page(sp, ktok0) * C::SROWB;
#pragma unroll
        for (int c = 0; c < 4; ++c) kb.ksc[c] = ld4_kv(srow + 4 * c * C::SROWB);  // byte lg is used
    }
    if constexpr (C::SC == SC_TOKEN && !C::PF) {
        const long off = ((long)sp.tpage * a.num_kv_heads * PG + slot_in_page(sp, 16 * lg)) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 kv4 = ld16(cx.ksbase + off + 16 * i), vv4 = ld16(cx.vsbase + off + 16 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // element first, then reinterpret: bit-casting a vector
                // element expression directly yields element 0 with this clang
                const uint32_t kw = kv4[j], vw = vv4[j];
                kb.tks[4 * i + j] = __builtin_bit_cast(float, kw);
                kb.tvs[4 * i + j] = __builtin_bit_cast(float, vw);
            }
        }
    }
}

// Whole-line K loads, once landed: lane 2p holds the low halves (bytes
// 128L + [0, 64) of a row) of tokens t(2p) and t(2p) + 1, lane 2p + 1 the high
// halves of the same two tokens. Exchanging the second register of the even
// lane with the first of the odd lane leaves each lane with its own token's
// bytes, as the MFMA operand layout of KBuf::k expects. The partner lane
// (ln ^ 1) is read with the DPP quad permutation [1, 0, 3, 2].
template <class C>
PA_DEV void fix_k(const Ctx& cx, KBuf<C>& kb) {
    if constexpr (C::KLINE) {
        constexpr int kSwapPairs = 0xB1;  // quad_perm [1, 0, 3, 2]: lane ^ 1
        const bool odd = cx.ln & 1;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int L = 0; L < C::KLOADS / 2; ++L) {
                u32x4& lo = kb.k[c][2 * L];
                u32x4& hi = kb.k[c][2 * L + 1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t x = lo[j], y = hi[j];
                    const uint32_t px = __builtin_amdgcn_mov_dpp((int)x, kSwapPairs, 0xF, 0xF, true);
                    const uint32_t py = __builtin_amdgcn_mov_dpp((int)y, kSwapPairs, 0xF, 0xF, true);
                    lo[j] = odd ? py : x;
                    hi[j] = odd ? y : px;
                }
            }
    }
}

// Whole-stage prefetch: per-token K and V scales of the slice by LDS DMA. Lane
// l fetches those of slice token l, which land at bytes [4l, 4l + 4) of the
// K half (slds) and of the V half (slds + 256). Scales of heads that share a
// page lie in one line, so the loads are not nontemporal.
template <class C>
PA_DEV void load_scales_dma(const TileArgs& a, const Ctx& cx, const SlicePages<C>& sp, char* slds) {
    const int l = cx.lane;
    // several pages per slice only with 16-token pages, where token l lies in
    // this lane's score page (tokens 16 lg + [0, 16))
    static_assert(C::NPC == 1 || C::PG == 16, "page of token l");
    const int pg = C::NPC == 1 ? sp.pg[0] : sp.tpage;
    const long off = ((long)pg * a.num_kv_heads * C::PG + slot_in_page(sp, l)) * 4;
    __builtin_amdgcn_global_load_lds((const void*)(cx.ksbase + off), (__attribute__((address_space(3))) void*)(slds),
                                     4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(cx.vsbase + off),
                                     (__attribute__((address_space(3))) void*)(slds + 256), 4, 0, 0);
}

// This lane's 16 K and V scales (slice tokens 16 lg + [0, 16)) from the scale
// block of a landed slice. slds is restrict-qualified: the next slice's DMA is
// in flight into the other block, and the full wait at the top of the slice
// already covers this one.
template <class C>
PA_DEV void read_scales_lds(const Ctx& cx, const char* __restrict__ slds, KBuf<C>& kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(slds + 64 * cx.lg + 16 * i);
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(slds + 256 + 64 * cx.lg + 16 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kb.tks[4 * i + j] = k4[j];
            kb.tvs[4 * i + j] = v4[j];
        }
    }
}

// Whole-stage prefetch: wait until every load issued so far has landed.
PA_DEV void full_wait() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_sched_barrier(0);
}

// Before a slice's V DMA: wait for everything outstanding (this slice's K).
// The compiler does not count LDS DMA instructions when it computes its own
// waits, so the wait it would put before QK for K loads issued ahead of the
// DMA is vmcnt(0), which also waits for the DMA just issued; waiting here
// instead lets the V transfer overlap QK.
template <class C>
PA_DEV void dma_fence() {
    if constexpr (C::VDMA) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <class C>
PA_DEV void load_v(const TileArgs& a, const Ctx& cx, const SlicePages<C>& sp, VBuf<C>& vb, char* vlds) {
    constexpr int PG = C::PG;
    const int ln = cx.ln, lg = cx.lg, lane = cx.lane;
    if constexpr (C::VDMA) {
        // instruction i fills LDS bytes [1024 i, 1024 i + 1024) of the wave's
        // tile: rows i * RPI + lane / CPR, chunk position lane % CPR; whole rows
        // per lane group, so the loads are nontemporal
        constexpr int RPI = 64 / C::CPR;
#pragma unroll
        for (int i = 0; i < C::CPR; ++i) {
            const int r = i * RPI + lane / C::CPR;
            const int c = (lane % C::CPR) ^ vswz<C>(r);
            const int vpage = sp.pg[C::NPC == 1 ? 0 : (i * RPI) / PG];  // uniform per instruction
            const long row = (long)vpage * a.num_kv_heads * PG + slot_in_page(sp, r);
            __builtin_amdgcn_global_load_lds((const void*)(cx.vbase + row * C::ROWB + 16 * c),
                                             (__attribute__((address_space(3))) void*)(vlds + 1024 * i), 16, 0,
                                             kLoadNontemporal);
        }
        // nothing moves across: the wait before PV counts the vector-memory
        // instructions issued after these
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (C::STAGE_V) {
        // step s stages slice tokens 16*(e>>3) + 8s + (e&7), e in [0, 32)
        const int vseg = lane % C::LPR;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < C::IPS; ++i) {
                const int e = i * C::TPI + lane / C::LPR;
                const int t = 16 * (e >> 3) + 8 * s + (e & 7);
                // page of token t: e >> 3 is the same for every lane of instruction i
                const int vpage = sp.pg[C::NPC == 1 ? 0 : ((i * C::TPI) >> 3) * 16 / PG];
                const long row = (long)vpage * a.num_kv_heads * PG + slot_in_page(sp, t);
                vb.v[s][i] = ld16_kv(cx.vbase + row * C::ROWB + 16 * vseg);
                if constexpr (C::KV == KV_MXFP4) vb.vsc[s][i] = ld4_kv(cx.vsbase + row * C::SROWB);  // byte vseg is used
            }
        // keep these loads at the top of the slice, ahead of QK: left alone, the
        // scheduler sinks them below QK, right before the staging that waits
        // for them, and the slice then pays the whole V latency
        if constexpr (C::PIN_V) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (C::VT) {
        // lane (d = 16dt + ln, lg) holds slice tokens 16*lg + [0, 16) of row d
        constexpr int VTW = C::ESZ == 2 ? 2 : 1;
        const char* vcol = cx.vbase + (long)sp.tpage * a.num_kv_heads * C::PAGE_BYTES_HEAD +
                           (long)slot_in_page(sp, 16 * lg) * C::ESZ;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int w = 0; w < VTW; ++w) vb.vt[dt][w] = ld16(vcol + (long)(16 * dt + ln) * PG * C::ESZ + 16 * w);
    }
}

// QK, scale, mask, online softmax (base 2) -> P^T fragments.
// qlds (QLDS instances): the query fragments in LDS, fragment (nt, ks) of lane
// l at byte 16 ((nt KSTEPS + ks) 64 + l); restrict-qualified, as the slice's V
// DMA is in flight while they are read.
template <class C, bool MASK>
PA_DEV void qk_softmax(const TileArgs& a, const Ctx& cx, const QFrag<C>& qf, const KBuf<C>& kb, State<C>& st,
                       PFrag<C>& pf, int cb, const char* __restrict__ qlds = nullptr) {
    constexpr int NT = C::NT;
    const int lg = cx.lg;
    // S^T[token][row]; acc[c][nt][j] <-> slice token 16*lg + 4c + j, row 16nt + ln
    f32x4 acc[4][NT];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if constexpr (C::QLDS && C::KV == KV_BF16) {
#pragma unroll
                for (int ks = 0; ks < C::KSTEPS; ++ks) {
                    const u32x4 q = *reinterpret_cast<const u32x4*>(qlds + 16 * ((nt * C::KSTEPS + ks) * 64 + cx.lane));
                    s = mfma_bf16(as_bf16x8(kb.k[c][ks]), as_bf16x8(q), s);
                }
            } else if constexpr (C::QLDS) {
#pragma unroll
                for (int u = 0; u < C::KLOADS; ++u) {
                    const u32x4 q0 = *reinterpret_cast<const u32x4*>(qlds + 16 * ((nt * C::KSTEPS + 2 * u) * 64 + cx.lane));
                    const u32x4 q1 =
                        *reinterpret_cast<const u32x4*>(qlds + 16 * ((nt * C::KSTEPS + 2 * u + 1) * 64 + cx.lane));
                    s = mfma_bf16(fp8x8_to_bf16x8(kb.k[c][u][0], kb.k[c][u][1]), as_bf16x8(q0), s);
                    s = mfma_bf16(fp8x8_to_bf16x8(kb.k[c][u][2], kb.k[c][u][3]), as_bf16x8(q1), s);
                }
            } else if constexpr (C::MXS) {
                i32x8 ka = {(int)kb.k[c][0][0], (int)kb.k[c][0][1], (int)kb.k[c][0][2], (int)kb.k[c][0][3], 0, 0, 0, 0};
                s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qf.q8[nt], s, 4, 0, 0,
                                                                     (int)((kb.ksc[c] >> (8 * lg)) & 0xFFu), 0,
                                                                     qf.qsc[nt]);
            } else if constexpr (C::KV == KV_MXFP4) {
                // K widened exactly: dword st holds d = 32g + 8st + [0, 8) times its block scale
                const float ksf = e8m0_to_f32((kb.ksc[c] >> (8 * lg)) & 0xFFu);
#pragma unroll
                for (int st = 0; st < C::KSTEPS; ++st)
                    s = mfma_bf16(as_bf16x8(fp4x8_to_bf16x8(kb.k[c][0][st], ksf)), qf.q[nt][st], s);
            } else if constexpr (C::KV == KV_BF16) {
#pragma unroll
                for (int ks = 0; ks < C::KSTEPS; ++ks) s = mfma_bf16(as_bf16x8(kb.k[c][ks]), qf.q[nt][ks], s);
            } else {
#pragma unroll
                for (int u = 0; u < C::KLOADS; ++u) {
                    s = mfma_bf16(fp8x8_to_bf16x8(kb.k[c][u][0], kb.k[c][u][1]), qf.q[nt][2 * u], s);
                    s = mfma_bf16(fp8x8_to_bf16x8(kb.k[c][u][2], kb.k[c][u][3]), qf.q[nt][2 * u + 1], s);
                }
            }
            acc[c][nt] = s;
            // QLDS: keep one 16-token group's K conversions and query reads
            // from being hoisted above the previous group's products
            if constexpr (C::QLDS) __builtin_amdgcn_sched_barrier(0);
        }

    const float sc = a.scale_log2 * cx.kscale;
    float tvs[16];
    if constexpr (C::SC == SC_TOKEN) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // per-token V scales of tokens at or past L, or before every row's
            // window, are staged as 0 (PR #7092, "Fix")
            const int tok = cb + 16 * lg + i;
            tvs[i] = (!MASK || (tok < cx.L && (!C::WIN || tok >= cx.s_lo))) ? kb.tvs[i] : 0.f;
        }
    }
    // The weights of N tile nt against the reference max muse: P (times the
    // per-token V scale) rounded to bf16 into pf, and their sum as l
    // accumulates it (returned in lsum).
#define PA_WEIGHTS(nt, muse, lsum)                                                                    \
    {                                                                                                 \
        uint32_t pw[8], plo[8];                                                                       \
        _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                               \
            float p[4];                                                                               \
            _Pragma("unroll") for (int j = 0; j < 4; ++j) p[j] = fast_exp2(acc[c][nt][j] - (muse));   \
            /* the weight sum: of P in fp32 where PV's weights are not the bf16 P itself */           \
            if constexpr (C::PSPLIT || C::SC == SC_TOKEN) lsum += (p[0] + p[1]) + (p[2] + p[3]);      \
            /* the PV weight: P times the token's V scale in fp32, rounded once */                    \
            if constexpr (C::SC == SC_TOKEN) {                                                        \
                _Pragma("unroll") for (int j = 0; j < 4; ++j) p[j] *= tvs[4 * c + j];                 \
            }                                                                                         \
            const uint32_t w0 = pack_bf16(p[0], p[1]), w1 = pack_bf16(p[2], p[3]);                    \
            if constexpr (C::PSPLIT) {                                                                \
                plo[2 * c] = pack_bf16(p[0] - bf16_lo(w0), p[1] - bf16_hi(w0));                       \
                plo[2 * c + 1] = pack_bf16(p[2] - bf16_lo(w1), p[3] - bf16_hi(w1));                   \
            } else if constexpr (C::SC != SC_TOKEN) {                                                 \
                /* the weight sum of exactly the rounded weights PV uses */                           \
                lsum += (bf16_lo(w0) + bf16_hi(w0)) + (bf16_lo(w1) + bf16_hi(w1));                    \
            }                                                                                         \
            pw[2 * c] = w0;                                                                           \
            pw[2 * c + 1] = w1;                                                                       \
        }                                                                                             \
        /* step s uses calls 2s (tokens 16lg + 8s + 0..3) and 2s + 1 (16lg + 8s + 4..7) */            \
        pf.hi[0][nt] = u32x4{pw[0], pw[1], pw[2], pw[3]};                                             \
        pf.hi[1][nt] = u32x4{pw[4], pw[5], pw[6], pw[7]};                                             \
        if constexpr (C::PSPLIT) {                                                                    \
            pf.lo[0][nt] = u32x4{plo[0], plo[1], plo[2], plo[3]};                                     \
            pf.lo[1][nt] = u32x4{plo[4], plo[5], plo[6], plo[7]};                                     \
        }                                                                                             \
    }
    float mloc[NT];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        mloc[nt] = -__builtin_inff();
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * lg + 4 * c + j;
                float x = acc[c][nt][j] * sc;
                if constexpr (C::SC == SC_TOKEN) x *= kb.tks[4 * c + j];
                // outside the row's causal / window range, or at or past L: -inf by a
                // select, never a multiply
                if (MASK) x = (cb + t >= cx.row_s[nt] && cb + t < cx.row_e[nt]) ? x : -__builtin_inff();
                else if (C::CAUSAL) x = cb + t < cx.row_e[nt] ? x : -__builtin_inff();
                acc[c][nt][j] = x;
                mloc[nt] = fmaxf(mloc[nt], x);
            }
        mloc[nt] = fmaxf(mloc[nt], shfl_xor(mloc[nt], 16));
        mloc[nt] = fmaxf(mloc[nt], shfl_xor(mloc[nt], 32));
        if constexpr (C::LAZY) {
            grow = grow || mloc[nt] > st.m[nt] + kRescaleLog2;
        } else {
            // re-based every slice
            const float mnew = fmaxf(st.m[nt], mloc[nt]);
            const float muse = (mnew == -__builtin_inff()) ? 0.f : mnew;
            const float alpha = fast_exp2(st.m[nt] - muse);
            st.m[nt] = mnew;
            float lsum = 0.f;
            PA_WEIGHTS(nt, muse, lsum)
            st.l[nt] = st.l[nt] * alpha + lsum;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) st.o[dt][nt] *= alpha;
        }
    }
    if constexpr (C::LAZY) {
        // Lazy rescaling: the reference max m of a row moves only on slices
        // where some row of the wave has seen its max grow past
        // m + kRescaleLog2 (one wave-uniform branch); otherwise the weights are
        // taken against the old m, at most 2^kRescaleLog2, and l and O are left
        // alone. (m, l, O) describe the same result either way; the per-element
        // rescale of O then runs on few slices instead of every one.
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float mnew = fmaxf(st.m[nt], mloc[nt]);
                const float alpha = fast_exp2(st.m[nt] - ((mnew == -__builtin_inff()) ? 0.f : mnew));
                st.m[nt] = mnew;
                st.l[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) st.o[dt][nt] *= alpha;
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float muse = (st.m[nt] == -__builtin_inff()) ? 0.f : st.m[nt];
            float lsum = 0.f;
            PA_WEIGHTS(nt, muse, lsum)
            st.l[nt] += lsum;
        }
    }
#undef PA_WEIGHTS
}

// Workgroup barrier ordering LDS accesses only. __syncthreads also waits for
// every outstanding global load, LDS DMA included; at a task switch that is
// the next task's first stage, whose latency the merge is meant to overlap.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier (the barrier builtin alone does not order memory); the
// wait makes this wave's LDS writes visible before it arrives.
PA_DEV void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), the other counters untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

PA_DEV void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// V operand preparation (boundary mask) and O^T[d][row] += V^T . P^T.
// VM_AFTER: vector-memory instructions issued between this slice's V DMA and
// this call (the next slice's K loads in the loop, none in the tail).
//
// The compiler's own wait for LDS written by DMA is vmcnt(0), which would also
// wait for the next slice's K loads; vlds is restrict-qualified here so that it
// leaves these reads alone, and the explicit wait below orders them after the
// DMA instead (the sched barriers pin the instruction order it counts on).
template <class C, bool MASK, int VM_AFTER>
PA_DEV void pv(const Ctx& cx, const VBuf<C>& vb, const PFrag<C>& pf, State<C>& st, int cb,
               char* __restrict__ vlds) {
    constexpr int NT = C::NT;
    const int ln = cx.ln, lg = cx.lg, lane = cx.lane;
    u32x4 vt[C::VT ? C::DT : 1][C::VT ? (C::ESZ == 2 ? 2 : 1) : 1];
    if constexpr (C::VT) {
        constexpr int VTW = C::ESZ == 2 ? 2 : 1;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int w = 0; w < VTW; ++w) vt[dt][w] = vb.vt[dt][w];
        if (MASK) {
            // keep only the bytes of tokens in [s_lo, L) (byte-granular, PR #7092 "Fix")
            const int valid = cx.L - (cb + 16 * lg);  // owned tokens among this lane's 16
            const int lead = C::WIN ? cx.s_lo - (cb + 16 * lg) : 0;  // of them, before every window
#pragma unroll
            for (int w = 0; w < VTW; ++w)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int first = (16 * w + 4 * j) / C::ESZ;  // first token of this dword
                    uint32_t mk = keep_bytes((valid - first) * C::ESZ);
                    if constexpr (C::WIN) mk &= ~keep_bytes((lead - first) * C::ESZ);
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) vt[dt][w][j] &= mk;
                }
        }
    }
    if constexpr (C::VDMA && !C::PF) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(VM_AFTER));  // this slice's V is in LDS
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if constexpr (C::STAGE_V) {
            // stage rows e of step s into the wave's LDS tile (bf16, row pitch VPITCH,
            // chunks placed by sv_row and sv_chunk); rows of tokens at or past L, or before
            // every row's window, are written as zeros
            const int vseg = lane % C::LPR;
            const int lrow = lane / C::LPR;  // < TPI
            constexpr int CPL = C::KV == KV_BF16 ? 1 : C::KV == KV_FP8 ? 2 : 4;  // bf16 chunks a lane
            char* dst = vlds + sv_row<C>(lrow) + sv_chunk<C>(CPL * vseg);
#pragma unroll
            for (int i = 0; i < C::IPS; ++i) {
                const int e = i * C::TPI + lrow;
                const int t = 16 * (e >> 3) + 8 * s + (e & 7);
                const bool ok = !MASK || (cb + t < cx.L && (!C::WIN || cb + t >= cx.s_lo));
                // row e = i TPI + lrow: sv_row(e) = sv_row(lrow) + this constant
                char* row = dst + (i * C::TPI) * C::VPITCH + ((i * C::TPI) >> 3) * C::VGRP;
                u32x4 raw = vb.v[s][i];
                if constexpr (C::KV == KV_BF16) {
                    if (!ok) raw = u32x4{0, 0, 0, 0};
                    *reinterpret_cast<u32x4*>(row) = raw;
                } else if constexpr (C::KV == KV_FP8) {
                    if (!ok) raw = u32x4{0, 0, 0, 0};
                    u32x2 a0 = fp8x4_to_bf16x4(raw[0]), a1 = fp8x4_to_bf16x4(raw[1]);
                    u32x2 a2 = fp8x4_to_bf16x4(raw[2]), a3 = fp8x4_to_bf16x4(raw[3]);
                    *reinterpret_cast<u32x4*>(row) = u32x4{a0[0], a0[1], a1[0], a1[1]};
                    *reinterpret_cast<u32x4*>(row + 16) = u32x4{a2[0], a2[1], a3[0], a3[1]};
                } else {
                    const float vsf = e8m0_to_f32((vb.vsc[s][i] >> (8 * vseg)) & 0xFFu);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x4 w = fp4x8_to_bf16x8(raw[j], vsf);
                        if (!ok) w = u32x4{0, 0, 0, 0};
                        *reinterpret_cast<u32x4*>(row + 16 * j) = w;
                    }
                }
            }
            wave_lds_sync();  // staged rows are read back by other lanes of the same wave
        }
        if constexpr (C::VDMA) {
            // The transposed reads of four d tiles are issued together, then
            // widened and multiplied, so that LDS latency overlaps the MFMAs.
            constexpr int CH = 4;
            typedef int i32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int d0 = 0; d0 < C::DT; d0 += CH) {
                u32x4 raw[CH];
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    const int dt = d0 + k;
                    if constexpr (C::KV == KV_BF16) {
                        // A lane (m, g) needs V[16g + 8s + e][16dt + m], e in [0, 8):
                        // two transposed reads; source lane ln reads row
                        // 16g + 8s + (ln >> 2) (+ 4), columns 16dt + 4 (ln & 3) + [0, 4)
                        const int r0 = 16 * lg + 8 * s + (ln >> 2);
                        const int c = 2 * dt + ((ln & 3) >> 1);
                        // vswz is the same for r0 and r0 + 4
                        const char* base = vlds + r0 * C::ROWB + 16 * (c ^ vswz<C>(r0)) + 8 * (ln & 1);
                        bf16x4 r0v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (__attribute__((address_space(3))) bf16x4*)(base));
                        bf16x4 r1v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (__attribute__((address_space(3))) bf16x4*)(base + 4 * C::ROWB));
                        raw[k] = __builtin_bit_cast(u32x4, bf16x8{r0v[0], r0v[1], r0v[2], r0v[3], r1v[0], r1v[1],
                                                                  r1v[2], r1v[3]});
                    } else {
                        // e4m3: one transposed byte read gives lane (m, g) the 8 bytes
                        // V[16g + 8s + e][16dt + m]; source lane ln reads 8 bytes of
                        // row 16g + 8s + (ln >> 1) at column 16dt + 8 (ln & 1)
                        const int r = 16 * lg + 8 * s + (ln >> 1);
                        const char* base = vlds + r * C::ROWB + 16 * (dt ^ vswz<C>(r)) + 8 * (ln & 1);
                        i32x2 b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(base));
                        raw[k] = u32x4{(uint32_t)b[0], (uint32_t)b[1], 0u, 0u};
                    }
                }
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    const int dt = d0 + k;
                    // element / byte e of this lane is token cb + 16g + 8s + e: zero
                    // those at or past L, and those before every row's window
                    // (PR #7092, "Fix")
                    const int valid = cx.L - (cb + 16 * lg + 8 * s);
                    const int lead = C::WIN ? cx.s_lo - (cb + 16 * lg + 8 * s) : 0;
                    bf16x8 va;
                    if constexpr (C::KV == KV_BF16) {
                        u32x4 w = raw[k];
                        if (MASK) {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                w[j] &= (valid > 2 * j && lead <= 2 * j ? 0x0000FFFFu : 0u) |
                                        (valid > 2 * j + 1 && lead <= 2 * j + 1 ? 0xFFFF0000u : 0u);
                        }
                        va = as_bf16x8(w);
                    } else {
                        uint32_t b0 = raw[k][0], b1 = raw[k][1];
                        if (MASK) {
                            b0 &= keep_bytes(valid) & ~keep_bytes(lead);
                            b1 &= keep_bytes(valid - 4) & ~keep_bytes(lead - 4);
                        }
                        va = fp8x8_to_bf16x8(b0, b1);
                    }
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        st.o[dt][nt] = mfma_bf16(va, as_bf16x8(pf.hi[s][nt]), st.o[dt][nt]);
                        if constexpr (C::PSPLIT) st.o[dt][nt] = mfma_bf16(va, as_bf16x8(pf.lo[s][nt]), st.o[dt][nt]);
                    }
                }
            }
            continue;
        }
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            bf16x8 va;
            if constexpr (C::STAGE_V) {
                // A lane (m = d offset, g) needs rows 8g + [0, 8) at column 16dt + m:
                // source lane ln reads row 8g + (ln >> 2) (+ 4), columns
                // 16dt + 4 (ln & 3) + [0, 4), i.e. half ln & 1 of chunk 2dt + ((ln & 3) >> 1)
                // sv_row(8 g + (ln >> 2)) and sv_chunk(2 dt + c), c < 2, as lane part
                // plus constant
                const char* base = vlds + (8 * lg + (ln >> 2)) * C::VPITCH + lg * C::VGRP + 16 * ((ln & 3) >> 1) +
                                   8 * (ln & 1) + sv_chunk<C>(2 * dt);
                bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(base));
                bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(base + 4 * C::VPITCH));
                va = bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
            } else if constexpr (C::ESZ == 2) {
                va = as_bf16x8(vt[dt][s]);
            } else {
                va = fp8x8_to_bf16x8(vt[dt][0][2 * s], vt[dt][0][2 * s + 1]);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                st.o[dt][nt] = mfma_bf16(va, as_bf16x8(pf.hi[s][nt]), st.o[dt][nt]);
                if constexpr (C::PSPLIT) st.o[dt][nt] = mfma_bf16(va, as_bf16x8(pf.lo[s][nt]), st.o[dt][nt]);
            }
        }
        if constexpr (C::STAGE_V) wave_lds_sync();  // the next step overwrites the tile
    }
}

// Tile range of one task: tiles [T0, T1) are read; [F0, F1) lie inside every
// row's range and run unmasked.
struct Range {
    int T0, T1, F0, F1;
};

// Set up task `idx` of the plan (plan-free: the task the block index names):
// sequence, KV head, partition, the sequence's context and the tile range.
//
// A planned launch reads its task (sequence, KV head | partition << 16, tile
// range) from the plan; a plan-free launch derives it from the block index
// (PR #7056, "Bandwidth": tasks follow from the block index): one task per
// (sequence, KV head) over all of its tiles, stored directly, or
// `uniform_parts` tasks of `part_tiles` tiles each, partition fastest.
//
// Tiles of the task: the task's range cut to the tiles any row reads (from
// the first row's window start to ceil(L / 256)). The first partition of a
// (sequence, KV head) starts at the device window's first tile whatever the
// plan says: a plan made from host lengths cuts the tiles before the host
// window, and a shorter device length moves the window earlier (the other
// partitions' ranges then still cover the rest). The window's first tiles and
// the causal and context boundary at the end run the masked variant.
// The task's own tile range before the cut, and the sequence's tile count.
struct TaskTiles {
    int tb, te, ntiles;
};

template <class C>
PA_DEV TaskTiles task_read(const TileArgs& a, int idx, Ctx& cx, int& part) {
    constexpr int PG = C::PG;
    int tb, te_task;
    if (a.plan_free) {
        const unsigned P = a.uniform_parts > 1 ? (unsigned)a.uniform_parts : 1u;
        const unsigned g = blockIdx.x / P;
        part = (int)(blockIdx.x % P);
        cx.b = (int)(g / (unsigned)a.num_kv_heads);
        cx.kvh = (int)(g % (unsigned)a.num_kv_heads);
        tb = part * a.part_tiles;
        te_task = (P == 1 || part == (int)P - 1) ? 0x7FFFFFFF : tb + a.part_tiles;
    } else {
        const int* task = a.tasks + 4 * idx;
        cx.b = uniform(task[0]);
        const int kp = uniform(task[1]);
        cx.kvh = kp & 0xFFFF;
        part = kp >> 16;
        tb = uniform(task[2]);
        te_task = uniform(task[3]);
    }
    int L = uniform(a.context_lens[cx.b]);
    L = L < 0 ? 0 : L;
    L = L > a.max_blocks * PG ? a.max_blocks * PG : L;
    cx.L = L;
    const int ntiles = (L + kTileTokens - 1) / kTileTokens;
    cx.npages = (L + PG - 1) / PG;
    cx.bt_row = a.block_tables + (long)cx.b * a.max_blocks;
    cx.kbase = reinterpret_cast<const char*>(a.k) + (long)cx.kvh * C::PAGE_BYTES_HEAD;
    cx.vbase = reinterpret_cast<const char*>(a.v) + (long)cx.kvh * C::PAGE_BYTES_HEAD;
    if constexpr (C::SC == SC_TOKEN) {
        cx.ksbase = reinterpret_cast<const char*>(a.ks) + (long)cx.kvh * PG * 4;
        cx.vsbase = reinterpret_cast<const char*>(a.vs) + (long)cx.kvh * PG * 4;
    } else if constexpr (C::KV == KV_MXFP4) {
        cx.ksbase = reinterpret_cast<const char*>(a.ks) + (long)cx.kvh * PG * C::SROWB;
        cx.vsbase = reinterpret_cast<const char*>(a.vs) + (long)cx.kvh * PG * C::SROWB;
    } else {
        cx.ksbase = cx.vsbase = nullptr;
    }
    return TaskTiles{tb, te_task, ntiles};
}

template <class C>
PA_DEV Range task_range(const TileArgs& a, const TaskTiles& tt, Ctx& cx, int part) {
    constexpr int PG = C::PG;
    const int L = cx.L, tb = tt.tb, te_task = tt.te, ntiles = tt.ntiles;
    // Query row r of this lane (query token i = r / G) attends to
    // [row_s, row_e): e = L - qlen + i + 1 when causal, else L; s = e - window
    // with a sliding window, else 0.
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        if constexpr (C::ROWS) {
            const int r = 16 * nt + cx.ln;
            const int i = r < a.rows ? r / a.q_per_kv : a.qlen - 1;
            const int e = a.causal ? L - a.qlen + i + 1 : L;
            cx.row_e[nt] = e;
            cx.row_s[nt] = a.window > 0 ? e - a.window : 0;
        } else {
            cx.row_e[nt] = L;
            cx.row_s[nt] = 0;
        }
    }
    // smallest row end (causal-only instances select every score against its
    // row's end instead, so their unmasked tiles run to the last one)
    const int e_min = C::WIN ? max(0, a.causal ? L - a.qlen + 1 : L) : L;
    const int s_min = C::WIN && a.window > 0 ? max(0, e_min - a.window) : 0;
    const int s_max = C::WIN && a.window > 0 ? max(0, L - a.window) : 0;
    // plan-free partitions count their tiles from the window's first tile
    const int w0 = C::WIN && a.plan_free ? s_min / kTileTokens : 0;
    cx.s_lo = s_min;
    cx.pg_first = C::WIN ? min(s_min / PG, max(cx.npages - 1, 0)) : 0;
    Range r;
    r.T0 = part == 0 ? s_min / kTileTokens : max(tb + w0, s_min / kTileTokens);
    r.T1 = te_task == 0x7FFFFFFF ? ntiles : min(te_task + w0, ntiles);
    r.F0 = max(r.T0, (s_max + kTileTokens - 1) / kTileTokens);
    r.F1 = max(r.F0, min(r.T1, e_min / kTileTokens));
    return r;
}

template <class C>
PA_DEV Range task_setup(const TileArgs& a, int idx, Ctx& cx, int& part) {
    const TaskTiles tt = task_read<C>(a, idx, cx, part);
    return task_range<C>(a, tt, cx, part);
}

// Merge the four waves' (m, l, O) of a finished task through LDS in a fixed
// order and store its rows: directly in bf16 when its (sequence, KV head) has
// one partition, else as partition `part`'s partial (O times the per-tensor V
// scale, and the row's max and weight sum). LDS: obuf0 and obuf1 hold
// ROWS_PAD x OPITCH fp32 each, mlbuf 8 x ROWS_PAD fp32; nothing else is
// touched. Every wave calls it; wave 0 stores.
template <class C>
PA_DEV void finish_task(const TileArgs& a, const Ctx& cx, State<C>& st, int part, float vscale,
                        float* __restrict__ obuf0, float* __restrict__ obuf1, float* __restrict__ mlbuf) {
    constexpr int NT = C::NT, D = C::D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        st.l[nt] += shfl_xor(st.l[nt], 16);
        st.l[nt] += shfl_xor(st.l[nt], 32);
    }
    lds_barrier();  // every wave's last P*V has read its V tile
    float* mbuf = mlbuf;                   // [4][ROWS_PAD]
    float* lbuf = mlbuf + 4 * C::ROWS_PAD;  // [4][ROWS_PAD]
    if (cx.lg == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            mbuf[cx.wave * C::ROWS_PAD + 16 * nt + cx.ln] = st.m[nt];
            lbuf[cx.wave * C::ROWS_PAD + 16 * nt + cx.ln] = st.l[nt];
        }
    }
    lds_barrier();
    float Mrow[NT], Lrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + cx.ln;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, mbuf[w * C::ROWS_PAD + r]);
        float Lt = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = mbuf[w * C::ROWS_PAD + r];
            Lt += (M == -__builtin_inff()) ? 0.f : fast_exp2(mw - M) * lbuf[w * C::ROWS_PAD + r];
        }
        const float f = (M == -__builtin_inff()) ? 0.f : fast_exp2(st.m[nt] - M);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) st.o[dt][nt] *= f;
        Mrow[nt] = M;
        Lrow[nt] = Lt;
    }
    auto obuf_at = [&](int buf, int nt, int dt) -> float* {
        return (buf ? obuf1 : obuf0) + (16 * nt + cx.ln) * C::OPITCH + 16 * dt + 4 * cx.lg;
    };
    if (cx.wave >= 2) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4*>(obuf_at(cx.wave - 2, nt, dt)) = st.o[dt][nt];
    }
    lds_barrier();
    if (cx.wave < 2) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) st.o[dt][nt] += *reinterpret_cast<f32x4*>(obuf_at(cx.wave, nt, dt));
    }
    lds_barrier();
    if (cx.wave == 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4*>(obuf_at(0, nt, dt)) = st.o[dt][nt];
    }
    lds_barrier();
    if (cx.wave != 0) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) st.o[dt][nt] += *reinterpret_cast<f32x4*>(obuf_at(0, nt, dt));

    // partitions of this (sequence, KV head) and its first partial unit
    const int pair = cx.b * a.num_kv_heads + cx.kvh;
    int nparts, unit0;
    if (a.plan_free) {
        nparts = a.uniform_parts > 1 ? a.uniform_parts : 1;
        unit0 = pair * nparts;
    } else {
        nparts = a.seq_parts[2 * pair];
        unit0 = a.seq_parts[2 * pair + 1];
    }
    const int Hq = a.num_kv_heads * a.q_per_kv;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + cx.ln;
        if (r >= a.rows) continue;
        if (nparts <= 1) {
            const float inv = (Lrow[nt] > 0.f) ? vscale / Lrow[nt] : 0.f;
            const long orow = ((long)cx.b * a.qlen + r / a.q_per_kv) * Hq + (long)cx.kvh * a.q_per_kv + r % a.q_per_kv;
            char* op = reinterpret_cast<char*>(a.out) + orow * D * 2;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const f32x4 o = st.o[dt][nt];
                u32x2 w = {pack_bf16(o[0] * inv, o[1] * inv), pack_bf16(o[2] * inv, o[3] * inv)};
                *reinterpret_cast<u32x2*>(op + 2 * (16 * dt + 4 * cx.lg)) = w;
            }
        } else {
            const long prow = ((long)unit0 + part) * a.rows + r;
            float* po = a.part_o + prow * D;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * cx.lg) = st.o[dt][nt] * vscale;
            if (cx.lg == 0) {
                a.part_ml[2 * prow] = Mrow[nt];
                a.part_ml[2 * prow + 1] = Lrow[nt];
            }
        }
    }
}

template <class C>
__global__ __launch_bounds__(kTileThreads, C::MINB) void pa_tile_kernel(const TileArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM_ALLOC];

    Ctx cx;
    cx.lane = threadIdx.x & 63;
    cx.wave = uniform(threadIdx.x >> 6);
    cx.ln = cx.lane & 15;
    cx.lg = cx.lane >> 4;
    int part;
    const TaskTiles tt = task_read<C>(a, blockIdx.x, cx, part);
    cx.kscale = 1.f;
    float vscale = 1.f;
    if constexpr (C::SC == SC_TENSOR) {
        cx.kscale = *reinterpret_cast<const float*>(a.ks);
        vscale = *reinterpret_cast<const float*>(a.vs);
    }
    QFrag<C> qf;
    load_q<C>(a, cx, qf);
    // (initialised here rather than in a helper taking a reference, which
    // costs the transposed-V instances 30 registers and spills)
    State<C> st;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        st.m[nt] = -__builtin_inff();
        st.l[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) st.o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    char* vlds = smem + cx.wave * C::WAVE_LDS;
    char* qlds = smem + 4 * C::WAVE_LDS;
    if constexpr (C::QLDS) {
        // one copy of the query fragments for the workgroup (the same for every wave)
        if (cx.wave == 0) {
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int ks = 0; ks < C::KSTEPS; ++ks)
                    *reinterpret_cast<u32x4*>(qlds + 16 * ((nt * C::KSTEPS + ks) * 64 + cx.lane)) =
                        __builtin_bit_cast(u32x4, qf.q[nt][ks]);
        }
        __syncthreads();
    }
    const Range rg = task_range<C>(a, tt, cx, part);
    const int T0 = rg.T0, T1 = rg.T1, F0 = rg.F0, F1 = rg.F1;
    using Masked = BoolTag<true>;
    using Full = BoolTag<false>;
    if constexpr (C::PF) {
        if (T1 > T0) {
            // stage = K (registers), V tile and scale block (LDS) of one slice;
            // stage(tile + 1) is issued right after the wait for stage(tile)
            constexpr int BUF = C::VSTAGE_BYTES + C::SCALE_BYTES;
            int cb = T0 * kTileTokens + 64 * cx.wave;
            PageCache<C> pc;
            page_cache_fill<C>(a, cx, pc, T0);
            SlicePages<C> sp = slice_pages<C>(a, cx, pc, T0);
            char* vcur = vlds;
            char* vnext = vlds + BUF;
            KBuf<C> kcur, knext;
            VBuf<C> vb;
            load_v<C>(a, cx, sp, vb, vcur);
            load_scales_dma<C>(a, cx, sp, vcur + C::VSTAGE_BYTES);
            load_k<C>(a, cx, sp, knext);
            int tile = T0;
            auto step = [&](auto mask_tag) {
                constexpr bool M = decltype(mask_tag)::value;
                full_wait();
                kcur = knext;
                sp = slice_pages<C>(a, cx, pc, tile + 1);
                load_v<C>(a, cx, sp, vb, vnext);
                load_scales_dma<C>(a, cx, sp, vnext + C::VSTAGE_BYTES);
                load_k<C>(a, cx, sp, knext);
                // the whole next stage is issued before this slice computes
                __builtin_amdgcn_sched_barrier(0);
                read_scales_lds<C>(cx, vcur + C::VSTAGE_BYTES, kcur);
                PFrag<C> pf;
                qk_softmax<C, M>(a, cx, qf, kcur, st, pf, cb);
                pv<C, M, 0>(cx, vb, pf, st, cb, vcur);
                char* t = vcur;
                vcur = vnext;
                vnext = t;
                cb += kTileTokens;
                ++tile;
            };
            if constexpr (C::WIN)
                for (; tile < F0 && tile + 1 < T1;) step(Masked{});
            for (; tile < F1 && tile + 1 < T1;) step(Full{});
            if constexpr (C::WIN)
                for (; tile + 1 < T1;) step(Masked{});
            full_wait();
            kcur = knext;
            read_scales_lds<C>(cx, vcur + C::VSTAGE_BYTES, kcur);
            PFrag<C> pf;
            qk_softmax<C, true>(a, cx, qf, kcur, st, pf, cb);
            pv<C, true, 0>(cx, vb, pf, st, cb, vcur);
        }
    } else if (T1 > T0) {
        // Loads run one stage ahead: V(j) is issued at the top of iteration j
        // (right after PV(j - 1)), K(j + 1) right after QK(j). Every load of a
        // loop is unconditional and each loop test comes after PV, so the waits
        // before QK and PV cover exactly the loads of the current slice, never
        // the prefetch in flight. The last tile runs after the loops with its
        // own V loads, masked (a no-op on a full tile).
        int cb = T0 * kTileTokens + 64 * cx.wave;
        PageCache<C> pc;
        page_cache_fill<C>(a, cx, pc, T0);
        SlicePages<C> sp = slice_pages<C>(a, cx, pc, T0);
        KBuf<C> kb;
        VBuf<C> vb;
        load_k<C>(a, cx, sp, kb);
        int tile = T0;
        // one tile with a successor: V(tile), QK, K(tile + 1), PV
        auto step = [&](auto mask_tag) {
            constexpr bool M = decltype(mask_tag)::value;
            dma_fence<C>();
            load_v<C>(a, cx, sp, vb, vlds);
            PFrag<C> pf;
            fix_k<C>(cx, kb);
            qk_softmax<C, M>(a, cx, qf, kb, st, pf, cb, qlds);
            sp = slice_pages<C>(a, cx, pc, tile + 1);
            load_k<C>(a, cx, sp, kb);
            pv<C, M, C::KVMEM>(cx, vb, pf, st, cb, vlds);
            cb += kTileTokens;
            ++tile;
        };
        if constexpr (C::WIN)
            for (; tile < F0 && tile + 1 < T1;) step(Masked{});  // window head
        for (; tile < F1 && tile + 1 < T1;) step(Full{});        // the bulk
        if constexpr (C::WIN)
            for (; tile + 1 < T1;) step(Masked{});               // causal boundary
        dma_fence<C>();
        load_v<C>(a, cx, sp, vb, vlds);
        PFrag<C> pf;
        fix_k<C>(cx, kb);
        qk_softmax<C, true>(a, cx, qf, kb, st, pf, cb, qlds);
        pv<C, true, 0>(cx, vb, pf, st, cb, vlds);
    }
    // the V tiles are free once every wave is past its last P*V (the merge's
    // first barrier)
    float* obuf = reinterpret_cast<float*>(smem);  // [2][ROWS_PAD][OPITCH], then [8][ROWS_PAD]
    finish_task<C>(a, cx, st, part, vscale, obuf, obuf + C::ROWS_PAD * C::OPITCH, obuf + 2 * C::ROWS_PAD * C::OPITCH);
}

// ------------------------------------------------------------- merge kernel

PA_DEV float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
    return v;
}
PA_DEV float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += shfl_xor(v, m);
    return v;
}

// One wave per output row (b, i, h) of a (sequence, KV head) with more than
// one partition (at most 64): M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p O_p / sum_p w_p l_p, summed in partition order (PR #7056,
// "Bandwidth": the partition reducer). Lane p reads partition p's (m, l); the
// weighted sum of the O_p rows then runs over p with D/64 elements per lane.
// The O rows of the first kMergePre partitions are loaded together with the
// (m, l) pairs, since they depend only on the partition table: the kernel then
// waits on memory twice (table, then partials) rather than three times.
template <int D>
__global__ __launch_bounds__(64) void pa_merge_kernel(const TileArgs a) {
    const int lane = threadIdx.x;
    const int Hq = a.num_kv_heads * a.q_per_kv;
    const long total = (long)a.num_seqs * a.qlen * Hq;
    const long R = blockIdx.x;
    if (R >= total) return;
    const int b = (int)(R / ((long)a.qlen * Hq));
    const int rem = (int)(R % ((long)a.qlen * Hq));
    const int i = rem / Hq, h = rem % Hq;
    const int kvh = h / a.q_per_kv;
    const int r = i * a.q_per_kv + h % a.q_per_kv;
    const int pair = b * a.num_kv_heads + kvh;
    // the row's (sequence, KV head) is the same for the whole wave
    const int P = uniform(a.plan_free ? a.uniform_parts : a.seq_parts[2 * pair]);
    if (P <= 1) return;
    const long unit0 = uniform(a.plan_free ? pair * P : a.seq_parts[2 * pair + 1]);
    const long stride = a.rows;  // rows between consecutive partitions
    const long prow0 = unit0 * a.rows + r;
    constexpr int PER = D / 64;
    constexpr int kMergePre = 16;
    const float* po = a.part_o + prow0 * D + PER * lane;
    using Row = typename std::conditional<PER == 4, f32x4, f32x2>::type;  // this lane's PER elements
    static_assert(PER == 2 || PER == 4, "head_dim 128 or 256");
    Row pre[kMergePre];
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) {
        pre[u] = Row{};
        if (u < P) pre[u] = *reinterpret_cast<const Row*>(po + u * stride * D);
    }
    float m = -__builtin_inff(), l = 0.f;
    if (lane < P) {
        const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * (prow0 + lane * stride));
        m = ml[0];
        l = ml[1];
    }
    const float M = wave_max(m);
    const float w = (lane < P && M != -__builtin_inff()) ? fast_exp2(m - M) : 0.f;
    const float den = wave_sum(w * l);
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) {
        if (u < P) {
            const float wp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] += wp * pre[u][k];
        }
    }
    int p = kMergePre;
    for (; p + 4 <= P; p += 4) {
        float v[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < PER; ++k) v[u][k] = po[(p + u) * stride * D + k];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float wp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), p + u));
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] += wp * v[u][k];
        }
    }
    for (; p < P; ++p) {
        const float wp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), p));
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] += wp * po[p * stride * D + k];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    char* op = reinterpret_cast<char*>(a.out) + R * D * 2 + 2 * PER * lane;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(op) = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
        *reinterpret_cast<u32x2*>(op) = u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
    }
}

// ---------------------------------------------------------------- dispatch

using TileFn = void (*)(const TileArgs);

struct Entry {
    KernelKey key;
    TileFn fn;
};

// Kernel instances are compiled in shards (PA_SHARD 0..4, one object file
// each, built in parallel); without PA_SHARD one object holds them all.
//   0: bf16 and MXFP4, plain decode      1: bf16 with causal rows / a window
//   2: e4m3 caches, plain decode         3: e4m3 with a window (or causal rows)
//   4: e4m3 with per-token scales, causal rows without a window
// Shard 0 also holds the merge kernel and the dispatch functions.
#ifndef PA_SHARD
#define PA_SHARD -1
#endif
#define PA_IN_SHARD(n) (PA_SHARD == -1 || PA_SHARD == (n))

#define PA_E(KV, SC, VT, D, PG, NT, QF, W) PA_EM(KV, SC, VT, D, PG, NT, QF, 0, W)
#define PA_EM(KV, SC, VT, D, PG, NT, QF, MXS, W) \
    {{KV, SC, VT, D, PG, NT, QF, MXS, W}, &pa_tile_kernel<Cfg<KV, SC, VT, D, PG, NT, QF, MXS, W>>}
#define PA_PG(KV, SC, VT, D, NT, W) \
    PA_E(KV, SC, VT, D, 16, NT, 0, W), PA_E(KV, SC, VT, D, 64, NT, 0, W), PA_E(KV, SC, VT, D, 128, NT, 0, W)
#define PA_NT(KV, SC, VT, D, W) PA_PG(KV, SC, VT, D, 1, W), PA_PG(KV, SC, VT, D, 2, W)
#define PA_D(KV, SC, VT, W) PA_NT(KV, SC, VT, 128, W), PA_PG(KV, SC, VT, 128, 4, W), PA_NT(KV, SC, VT, 256, W)
#define PA_VT(KV, SC, W) PA_D(KV, SC, 0, W), PA_D(KV, SC, 1, W)

#if PA_IN_SHARD(0)
extern const Entry kShard0[] = {
    PA_VT(KV_BF16, SC_NONE, 0),
    PA_EM(KV_MXFP4, SC_NONE, 0, 128, 128, 1, 0, 0, 0),
    PA_EM(KV_MXFP4, SC_NONE, 0, 128, 128, 1, 1, 0, 0),
    PA_EM(KV_MXFP4, SC_NONE, 0, 128, 128, 1, 0, 1, 0),
    PA_EM(KV_MXFP4, SC_NONE, 0, 128, 128, 1, 1, 1, 0),
};
extern const int kShard0Size = sizeof(kShard0) / sizeof(kShard0[0]);
#endif
#if PA_IN_SHARD(1)
extern const Entry kShard1[] = {PA_VT(KV_BF16, SC_NONE, 1)};
extern const int kShard1Size = sizeof(kShard1) / sizeof(kShard1[0]);
#endif
#if PA_IN_SHARD(2)
extern const Entry kShard2[] = {PA_VT(KV_FP8, SC_TENSOR, 0), PA_VT(KV_FP8, SC_TOKEN, 0)};
extern const int kShard2Size = sizeof(kShard2) / sizeof(kShard2[0]);
#endif
#if PA_IN_SHARD(3)
extern const Entry kShard3[] = {PA_VT(KV_FP8, SC_TENSOR, 1), PA_VT(KV_FP8, SC_TOKEN, 1)};
extern const int kShard3Size = sizeof(kShard3) / sizeof(kShard3[0]);
#endif

#if PA_IN_SHARD(4)
extern const Entry kShard4[] = {PA_VT(KV_FP8, SC_TOKEN, 2)};
extern const int kShard4Size = sizeof(kShard4) / sizeof(kShard4[0]);
#endif

#if PA_IN_SHARD(0)
extern const Entry kShard1[], kShard2[], kShard3[], kShard4[];
extern const int kShard1Size, kShard2Size, kShard3Size, kShard4Size;

static const Entry* find_entry(const KernelKey& k) {
    const Entry* tables[5] = {kShard0, kShard1, kShard2, kShard3, kShard4};
    const int sizes[5] = {kShard0Size, kShard1Size, kShard2Size, kShard3Size, kShard4Size};
    for (int t = 0; t < 5; ++t)
        for (int i = 0; i < sizes[t]; ++i) {
            const Entry& e = tables[t][i];
            if (e.key.kv == k.kv && e.key.scale == k.scale && e.key.vt == k.vt && e.key.head_dim == k.head_dim &&
                e.key.page == k.page && e.key.ntiles_n == k.ntiles_n && e.key.q_fp8 == k.q_fp8 &&
                e.key.mx_scaled == k.mx_scaled && e.key.win == k.win)
                return &e;
        }
    return nullptr;
}

static TileFn find(const KernelKey& k) {
    const Entry* e = find_entry(k);
    return e ? e->fn : nullptr;
}

bool have_tile_kernel(const KernelKey& key) { return find(key) != nullptr; }

int tile_blocks_per_cu(const KernelKey& key) {
    TileFn fn = find(key);
    if (!fn) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kTileThreads, 0) != hipSuccess) return 1;
    return n < 1 ? 1 : n;
}

hipError_t launch_tile(const KernelKey& key, const TileArgs& args, int num_tasks, hipStream_t stream) {
    TileFn fn = find(key);
    if (!fn) return hipErrorInvalidValue;
    if (num_tasks <= 0) return hipSuccess;
    hipLaunchKernelGGL(fn, dim3(num_tasks), dim3(kTileThreads), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_merge(const TileArgs& args, int head_dim, hipStream_t stream) {
    const long rows = (long)args.num_seqs * args.qlen * args.num_kv_heads * args.q_per_kv;
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    // one single-wave workgroup per row: the rows spread over four times as
    // many compute units as with four waves per workgroup (cold per call, fp8
    // per-token qlen 1 69.5 -> 69.2 us, MXFP4 at 2048 tokens 16.3 -> 16.2 us,
    // bf16 head_dim 256 with one 1024-token sequence 18.7 -> 18.4 us)
    const unsigned blocks = (unsigned)rows;
    if (head_dim == 128)
        hipLaunchKernelGGL(pa_merge_kernel<128>, dim3(blocks), dim3(64), 0, stream, args);
    else if (head_dim == 256)
        hipLaunchKernelGGL(pa_merge_kernel<256>, dim3(blocks), dim3(64), 0, stream, args);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
#endif  // PA_IN_SHARD(0)

}  // namespace pa
