// Matrix-core GEMM for gfx950 with direct-to-LDS loads and an S-stage LDS
// ring: D = alpha * op(A) * op(B) + beta * C, bf16 or fp32 operands, fp32
// accumulate, fp32 or bf16 out.  A workgroup of WM x WN waves computes one
// BM x BN output tile (the selected bf16 256x256 tile uses 8 waves, two per
// SIMD, so one wave's waits are covered by the other's matrix work).
//
// Same hierarchical tiling as mfma_gemm.hpp ("GEMM on NVIDIA GPUs: from a
// naive kernel to a tiled pipeline", section 4), with the load/compute
// overlap of its "load-compute overlap" part made deeper:
//
//  * Each operand tile of a K-step goes from global memory straight into LDS
//    with buffer_load_dwordx4 ... lds (lane l of a wave writes its 16 bytes at
//    the instruction's LDS base + 16*l), so no registers hold tiles in flight
//    and no VALU or LDS-write instructions are spent on staging.  Which global
//    16-byte chunk a lane fetches is chosen so the LDS image comes out in the
//    swizzled layout below.  One buffer resource per operand starts at the
//    workgroup's panel and ends where the stored matrix ends: a lane's offset
//    is its fixed in-step offset plus the step's, and reads past the matrix
//    return zero (buffer range checking).  Addresses need only element
//    alignment: gfx9+ runs in the unaligned access mode, where a 16-byte load
//    at a 2- or 4-byte aligned address is served whole.
//  * Operands keep their memory orientation in LDS.  A k-contiguous operand
//    (A with transA == N, B with transB == T) is stored [mn][k] in 16-byte
//    chunks with the chunk index XOR-swizzled by row, and its MFMA fragments
//    are read with ds_read_b128.  An mn-contiguous operand (A with T, B with N)
//    is stored [k][mn] with 32-byte blocks XOR-swizzled by a table indexed by
//    (k mod 4), and its
//    fragments are read with two ds_read_b64_tr_b16: within each 16-lane
//    group, lane r+4j supplies the address of (k0+j, mn0+4r..4r+3) and lane
//    4r+e receives element e of lanes r, r+4, r+8, r+12, i.e. four
//    consecutive k of column mn0+4r+e — exactly an MFMA operand slice.
//    Read addresses come from a few per-lane base registers plus
//    compile-time constants (FragAddr).
//  * S stages in separate __shared__ arrays (static indices keep the
//    compiler's LDS-DMA dependency tracking exact).  One barrier per stage:
//    before it each wave waits until the next stage's DMA has landed; after
//    it the DMA for a later step is issued into a buffer every wave has
//    finished reading, and the next stage's first fragments are read while
//    the MFMAs run.  The barrier sits either half way through the stage's
//    MFMAs (copying S-1 steps ahead into the previous step's buffer, S >= 3)
//    or before its last fragment step (copying S steps ahead into the
//    current buffer once this wave's reads of it are done, S >= 2).
//  * MFMA operands are swapped (B fragment first), so each lane's
//    accumulators hold 4 adjacent output columns of one row: the epilogue
//    writes 16-byte vectors.
//  * The ragged last K-step and the last step of edge tiles take a
//    register-staged path with per-element zero fill that writes the same
//    LDS layout (ds_write_b128); so does every step when the host finds a
//    panel whose byte offsets would not fit in 32 bits (ALIGNED == false).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "mfma_gemm.hpp"
#include "sk_ranges.hpp"

namespace dg {

// LATE_ selects where a step's barrier sits: false = half way through the
// step's fragment steps, copying the step S-1 ahead into the stage read one
// step earlier; true = before the step's last fragment step, once this wave's
// reads of the step have completed, copying the step S ahead into the stage
// just read.  The late barrier hides one more step of copy latency with the
// same number of stages, so two stages suffice.
//
// PAIR_ (late barrier only): PAIR_KC copies every k-contiguous operand two
// K-steps at a time into one of NP pair buffers holding 2*BK k per row, so
// each group of lanes fetches whole 128-byte lines where a BK = 32 bf16 step
// covers only half of each line (the other half would be requested again,
// from L2, one step later); an mn-contiguous operand keeps the S-stage ring
// (a round of slots, the least common multiple of S and 2*NP, is at most 6
// steps).  PAIR_BOTH_KC does so only when both operands
// are k-contiguous (measured: pairing pays there, and not when one operand
// is mn-contiguous), PAIR_ONE_KC only when the other one is mn-contiguous.
// A pair is copied at the barrier of the odd step that finishes the
// buffer's previous pair.
enum : int { PAIR_NONE = 0, PAIR_KC = 1, PAIR_BOTH_KC = 2, PAIR_ONE_KC = 3 };
//
// WPE_ > 0 asks the compiler for at least that many waves per SIMD, i.e.
// that many resident workgroups per compute unit for 4-wave workgroups
// (a register budget of 512 / WPE_ per lane).  NP_ = 2 or 3 pair buffers:
// with NP, a pair is copied 2*NP - 1 steps ahead of its first step.
template <int KIND_, int BM_, int BN_, int BK_, int WM_, int WN_, int S_, bool LATE_ = false,
          int PAIR_ = PAIR_NONE, int WPE_ = 0, int NP_ = 2>
struct DmaConfig {
    static constexpr int KIND = KIND_, BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, S = S_;
    static constexpr bool LATE = LATE_;
    static constexpr int PAIR = PAIR_;
    static constexpr int WPE = WPE_ > 0 ? WPE_ : 1;
    static constexpr int NP = NP_;
    static constexpr int AHEAD = LATE ? S : S - 1;  // steps between a copy and its use
    using T = typename MfmaShape<KIND>::T;
    static constexpr int ES = sizeof(T);
    static constexpr int VEC = 16 / ES;                // elements per 16-byte chunk
    static constexpr int FM = MfmaShape<KIND>::FM;
    static constexpr int ACC = MfmaShape<KIND>::ACC;
    static constexpr int KG = 64 / FM;                 // lane groups along k
    static constexpr int KSTEP = KG * VEC;             // k per fragment
    static constexpr int NKS = BK / KSTEP;             // fragment steps per stage
    static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MF = WTM / FM, NF = WTN / FM;
    // An operand tile's extent along mn as laid out in LDS: the next power of
    // two (a 192-wide tile occupies 256), so the XOR swizzles, which permute
    // chunk indices within a power-of-two row, and the 1 KiB-per-wave DMA
    // split hold for every tile width.  The padding is copied as zeros (or
    // as whatever the buffer range admits) and never read.
    static constexpr int pad_extent(int r)
    {
        int e = 1;
        while (e < r) e *= 2;
        return e;
    }
    static constexpr int A_BYTES = pad_extent(BM) * BK * ES, B_BYTES = pad_extent(BN) * BK * ES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // whether an operand that is (kc) k-contiguous is paired when the other
    // one is (other_kc)
    static constexpr bool pairs(bool kc, bool other_kc)
    {
        return kc && (PAIR == PAIR_KC || (PAIR == PAIR_BOTH_KC && other_kc) ||
                      (PAIR == PAIR_ONE_KC && !other_kc));
    }
    static constexpr int lds_for(bool a_kc, bool b_kc)
    {
        const bool pa = pairs(a_kc, b_kc), pb = pairs(b_kc, a_kc);
        return S * ((pa ? 0 : A_BYTES) + (pb ? 0 : B_BYTES)) +
               NP * 2 * ((pa ? A_BYTES : 0) + (pb ? B_BYTES : 0));
    }
    static constexpr int max2(int x, int y) { return x > y ? x : y; }
    // largest LDS footprint over the four operand orientations
    static constexpr int LDS_BYTES = max2(max2(lds_for(false, false), lds_for(false, true)),
                                          max2(lds_for(true, false), lds_for(true, true)));
    static constexpr int A_DMA = A_BYTES / (1024 * WAVES);  // DMA instructions per wave
    static constexpr int B_DMA = B_BYTES / (1024 * WAVES);
    static constexpr int DMA_PER_STAGE = A_DMA + B_DMA;
    static_assert(KIND == MFMA_BF16_32x32x16 || KIND == MFMA_BF16_16x16x32 ||
                      KIND == MFMA_F32_32x32x2,
                  "instruction kinds with a defined fragment mapping");
    static_assert(S >= (LATE ? 2 : 3) && S <= 5, "stage count");
    static_assert(PAIR == PAIR_NONE || LATE, "paired copies need the late barrier");
    static_assert(NP == 2 || NP == 3, "pair buffers");
    static_assert(NKS >= 2 && NKS % 2 == 0, "barrier sits between fragment steps");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "DMA split");
    static_assert(BM % (WM * FM) == 0 && BN % (WN * FM) == 0, "wave tile");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
    static_assert(DMA_PER_STAGE * (AHEAD - 1) < 64, "vmcnt range");
};

// XOR applied to the 16-byte chunk index of row k of an [k][mn] tile: {0, 4,
// 10, 14} for k mod 4 = 0..3.  A transposed fragment read touches 4 rows and,
// per 16 lanes, 2 adjacent chunks (32 bytes): with these masks the 4 rows'
// chunk pairs fill a 128-byte bank window exactly, and the two 16-lane groups
// of a 32-lane half (chunks 2 apart) fill a 256-byte window exactly.
__host__ __device__ constexpr int mn_swz(int k) { return (0x0E0A0400 >> (8 * (k & 3))) & 0xFF; }

// LDS layout of one operand tile.  R = rows of the tile in the mn direction,
// KD = k per row of a k-contiguous tile (BK, or 2*BK for a pair buffer).
template <class Cfg, int R, bool KC, int KD = Cfg::BK>
struct Layout {
    static constexpr int BK = KD;
    static constexpr int RP = Cfg::pad_extent(R);  // rows (KC) or row width in LDS
    static constexpr int CPR_K = BK / Cfg::VEC;   // chunks per [mn][k] row
    static constexpr int CPR_M = RP / Cfg::VEC;   // chunks per [k][mn] row
    static_assert(!KC || CPR_K == 4 || CPR_K == 8, "k-major swizzle");
    static_assert(KC || CPR_M >= 16, "mn-major swizzle needs >= 16 chunks per row");
    // XOR for row k of an [k][mn] tile: bf16 rows are read 4 at a time by the
    // transposing reads (table above); fp32 rows are read by 32-bit reads in
    // which the two half-waves take rows 4 apart, so rows with bit 2 of k set
    // move to the other 128-byte half of each 256-byte window.  With 16-wide
    // fragments the two 16-lane groups of a half-wave read the same chunks of
    // rows 8 apart (32-wide ones read chunks 2 apart of the same rows), so
    // rows with bit 3 of k set also swap chunk pairs (XOR 2), which puts the
    // two groups in one 256-byte window as with 32-wide fragments.
    __host__ __device__ static constexpr int mswz(int k)
    {
        if constexpr (Cfg::ES == 2) return mn_swz(k) ^ (Cfg::FM == 16 ? ((k >> 3) & 1) << 1 : 0);
        else return ((k >> 2) & 1) << 3;
    }
    // XOR for row mn of an [mn][k] tile.  A fragment read covers 32 (or 16)
    // consecutive rows at one or two chunks.  With 8 chunks per row the rows
    // swizzled by (r ^ r>>3) already spread every 16 lanes over all banks.
    // With 4 chunks per row (64-byte rows) measured bank-conflict counts on
    // gfx950 are zero for (r ^ r>>2) & 3 but four cycles per ds_read_b128 for
    // any swizzle that mixes in row bit 3, such as ((r>>1) ^ (r>>3)) & 3.
    __host__ __device__ static constexpr int kswz(int r)
    {
        if constexpr (CPR_K == 4) return (r ^ (r >> 2)) & 3;
        else return (r ^ (r >> 3)) & 7;
    }
    // byte offset of 16-byte chunk `chunk` in LDS row `row`
    __host__ __device__ static constexpr int off(int row, int chunk)
    {
        if constexpr (KC)
            return row * (CPR_K * 16) + ((chunk ^ kswz(row)) << 4);
        else
            return row * (CPR_M * 16) + ((chunk ^ mswz(row)) << 4);
    }
    static constexpr int ROWS = KC ? RP : BK;       // LDS rows
    static constexpr int CPR = KC ? CPR_K : CPR_M;  // chunks per LDS row
};

// Addresses of the MFMA operand fragments a wave reads from one LDS buffer
// of an operand (Layout<Cfg, R, KC, KD>), for a wave tile WT wide along mn
// and NWP wave positions along mn (wave tile w starts at mn = w * WT).
// Fragment (i, kk) is the FM x KSTEP operand slice of rows w*WT + i*FM ..
// +FM-1 at k-fragment kk of the buffer, read in NPC pieces: one ds_read_b128
// (k-contiguous), two transposing ds_read_b64_tr_b16 (bf16, mn-contiguous)
// or four 32-bit reads (fp32, mn-contiguous).
//
// The swizzles make a lane's offset a different permutation for some
// (i, kk, piece) combinations, but many combinations differ from one another
// by the same constant in every lane.  PLAN groups them at compile time,
// checking every lane and wave position: each group keeps one per-lane base
// register, and a read adds its combination's constant, which the LDS
// instruction's offset field absorbs.  So a wave needs a few address
// registers instead of one per combination and stage.
template <class Cfg, int R, bool KC, int KD, int WT, int NWP>
struct FragAddr {
    using L = Layout<Cfg, R, KC, KD>;
    static constexpr int FM = Cfg::FM, KG = Cfg::KG, KSTEP = Cfg::KSTEP, VEC = Cfg::VEC;
    static constexpr int NPC = KC ? 1 : (Cfg::ES == 2 ? 2 : 4);  // pieces per fragment
    static constexpr int NFRAG = WT / FM;
    static constexpr int NKSA = KD / KSTEP;
    static constexpr int NCOMBO = NFRAG * NKSA * NPC;
    static_assert(WT % FM == 0 && KD % KSTEP == 0, "fragment grid");
    __host__ __device__ static constexpr int combo(int i, int kk, int pc)
    {
        return (i * NKSA + kk) * NPC + pc;
    }

    // Byte offset of piece pc of fragment (i, kk) for `lane` of the wave
    // whose tile starts at mn index wmn0 (the MFMA operand lane mappings:
    // k-contiguous, lane l holds row l % FM, k-chunk l / FM; transposing
    // reads, lane r + 4j of each 16-lane group g addresses k-row j (+4 for the
    // second piece, +8 per group pair) at mn 4r (+16 for odd groups with
    // 32-wide fragments); fp32 32-bit reads, lane l holds mn l % 32 at k
    // 4 (l / 32) + piece).
    __host__ __device__ static constexpr int raw_off(int i, int kk, int pc, int lane, int wmn0)
    {
        const int mn0 = wmn0 + i * FM;
        if constexpr (KC) {
            return L::off(mn0 + lane % FM, kk * KG + lane / FM);
        } else if constexpr (Cfg::ES == 4) {
            const int mn = mn0 + (lane & 31);
            const int k = kk * KSTEP + 4 * (lane >> 5) + pc;
            return L::off(k, mn / VEC) + (mn % VEC) * 4;
        } else {
            const int g = lane >> 4, q = lane & 15, r = q & 3, j = q >> 2;
            int mn = 0, k = 0;
            if constexpr (FM == 32) {
                mn = mn0 + 16 * (g & 1) + 4 * r;
                k = kk * KSTEP + 8 * (g >> 1) + 4 * pc + j;
            } else {
                mn = mn0 + 4 * r;
                k = kk * KSTEP + 8 * g + 4 * pc + j;
            }
            return L::off(k, mn >> 3) + (mn & 7) * 2;
        }
    }

    struct Plan {
        int nbase = 0;
        int base_combo[NCOMBO] = {};  // the combination each base register is computed for
        int base_shift[NCOMBO] = {};  // ... plus this constant
        int cls[NCOMBO] = {};         // base register of each combination
        int delta[NCOMBO] = {};       // ... and its constant (>= 0)
    };
    __host__ __device__ static constexpr int off_of(int x, int lane, int wmn0)
    {
        return raw_off(x / (NKSA * NPC), (x / NPC) % NKSA, x % NPC, lane, wmn0);
    }
    // whether combinations x and y differ by one constant d in every lane and
    // wave position
    __host__ __device__ static constexpr bool same_class(int x, int y, int& d)
    {
        d = off_of(x, 0, 0) - off_of(y, 0, 0);
        for (int w = 0; w < NWP; ++w)
            for (int lane = 0; lane < 64; ++lane)
                if (off_of(x, lane, w * WT) - off_of(y, lane, w * WT) != d) return false;
        return true;
    }
    __host__ __device__ static constexpr Plan make()
    {
        Plan p{};
        for (int x = 0; x < NCOMBO; ++x) {
            int b = 0, d = 0;
            for (; b < p.nbase; ++b)
                if (same_class(x, p.base_combo[b], d)) break;
            if (b == p.nbase) {
                p.base_combo[b] = x;
                ++p.nbase;
                d = 0;
            }
            p.cls[x] = b;
            p.delta[x] = d;
        }
        for (int b = 0; b < p.nbase; ++b) {
            int lo = 0;
            for (int x = 0; x < NCOMBO; ++x)
                if (p.cls[x] == b && p.delta[x] < lo) lo = p.delta[x];
            p.base_shift[b] = lo;
            for (int x = 0; x < NCOMBO; ++x)
                if (p.cls[x] == b) p.delta[x] -= lo;
        }
        return p;
    }
    static constexpr Plan PLAN = make();
    static constexpr int NBASE = PLAN.nbase;
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (stride 0) over the bytes [base, base + nrec).  A 16-byte
// load through it returns zero for every 4-byte word that does not lie wholly
// below nrec, and touches no memory for it.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t nrec)
{
    const uint64_t a = reinterpret_cast<uintptr_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                 __builtin_amdgcn_readfirstlane((int)nrec), 0x00020000};
}

// PAIRED: the operand lives in pair buffers (k-contiguous only): a DMA copy
// covers two K-steps, register-staged copies one step into half `half`.
// WT, NWP: the wave tile's extent along mn and the wave positions along mn.
template <class Cfg, int R, bool KC, bool ALIGNED, bool PAIRED, int WT, int NWP>
struct DmaOperand {
    static_assert(!PAIRED || KC, "only k-contiguous operands are paired");
    static constexpr int KD = PAIRED ? 2 * Cfg::BK : Cfg::BK;  // k per buffer
    using L = Layout<Cfg, R, KC, KD>;
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC;
    static constexpr int ND = (L::RP * KD * Cfg::ES) / (1024 * Cfg::WAVES);  // DMA instructions per wave
    static constexpr int BYTES = L::RP * KD * Cfg::ES;                     // one buffer
    static constexpr int SCPR = KC ? Cfg::BK / VEC : R / VEC;          // chunks per row of one step
    static constexpr int CHUNKS = (KC ? R : Cfg::BK) * SCPR;           // chunks of one step
    static constexpr int GL = (CHUNKS + Cfg::THREADS - 1) / Cfg::THREADS;  // guarded loads per thread

    // Per-lane byte offsets of this lane's DMA chunks from the start of a step
    // (row = mn and chunks along k for KC, row = k and chunks along mn
    // otherwise).  The host keeps every offset within the panel below 2^32.
    // Chunks of the padding beyond R get an offset of 2^31: past the end of
    // any panel the buffer range reaches below 2 GiB they read as zero without
    // touching memory, and otherwise they fetch bytes of the matrix itself;
    // either way nothing reads them back.
    uint32_t voff[ND];

    __device__ __forceinline__ void init(int wave, int lane, int64_t ld)
    {
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const int pos = (wave * ND + d) * 1024 + lane * 16;  // byte position in the tile
            const int row = pos / (L::CPR * 16);
            const int pc = (pos % (L::CPR * 16)) >> 4;
            // invert the swizzle: which logical chunk lives at physical chunk pc
            int c;
            if constexpr (KC) c = pc ^ L::kswz(row);
            else c = pc ^ L::mswz(row);
            const bool pad = KC ? row >= R : c * VEC >= R;
            voff[d] = pad ? 0x80000000u : (uint32_t)(((int64_t)row * ld + c * VEC) * Cfg::ES);
        }
    }

    // Buffer resource of the panel: based at the panel start, with its range
    // ending where the stored matrix ends (`end`), so chunks of rows past the
    // matrix read as zero instead of touching memory.
    __device__ static __forceinline__ i32x4 panel_rsrc(const T* panel, const char* end)
    {
        const int64_t left = end - reinterpret_cast<const char*>(panel);
        return buffer_rsrc(panel, left > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)left);
    }

    // Byte offset of the step at k0 from the panel start.
    __device__ static __forceinline__ uint32_t step_bytes(int k0, int64_t ld)
    {
        return (uint32_t)((KC ? (int64_t)k0 : (int64_t)k0 * ld) * Cfg::ES);
    }

    // The d-th DMA copy of a step: 16 bytes per lane from the buffer into LDS at
    // the instruction's base + 16 * lane.  Issued through inline asm (the LDS
    // destination goes in as an m0 operand, so the compiler sets m0 itself): the
    // kernel orders these copies itself with explicit s_waitcnt vmcnt + s_barrier,
    // so the compiler's own (conservative) LDS-DMA tracking adds no waits; any
    // wait it inserts for its own loads can only become stronger because of these
    // extra outstanding operations.
    __device__ __forceinline__ void dma_one(int d, i32x4 rsrc, uint32_t kbytes, char* lds,
                                            int wave) const
    {
        uint32_t lds_base = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lds) + wave * ND * 1024);
        // Opaque to the optimizer, so each copy's m0 is one scalar add at its
        // use: hoisted out of the loop, the per-copy values of every stage
        // would each hold an SGPR and exhaust them.
        asm volatile("" : "+s"(lds_base));
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff[d] + kbytes), "s"(rsrc), "{m0}"(lds_base + d * 1024)
                     : "memory");
    }

    __device__ __forceinline__ void dma(i32x4 rsrc, uint32_t kbytes, char* lds, int wave) const
    {
#pragma unroll
        for (int d = 0; d < ND; ++d) dma_one(d, rsrc, kbytes, lds, wave);
    }

    // Register-staged copy of the step at k0 with zero fill outside
    // [0, rlim) x [0, K), into half `half` of a pair buffer when PAIRED.
    __device__ __forceinline__ void guarded(const T* panel, int64_t ld, int rlim, int k0, int K,
                                            char* lds, int tid, int half = 0) const
    {
        // in batches of GB chunks per thread, which bounds the registers this
        // path adds on top of the accumulators and fragments
        constexpr int GB_MAX = Cfg::WPE > 1 ? 1 : 4;
        constexpr int GB = GL < GB_MAX ? GL : GB_MAX;
#pragma unroll
        for (int i0 = 0; i0 < GL; i0 += GB) {
            u32x4 v[GB];
#pragma unroll
            for (int b = 0; b < GB; ++b) {
                const int q = tid + (i0 + b) * Cfg::THREADS;
                if ((CHUNKS % Cfg::THREADS != 0 || GL % GB != 0) && (i0 + b >= GL || q >= CHUNKS)) break;
                const int row = q / SCPR, c = q % SCPR;
                T e[VEC];
                if constexpr (KC) {   // row = mn, elements along k
                    const int k = k0 + c * VEC;
                    const T* src = panel + (int64_t)row * ld + k;
                    if (ALIGNED && row < rlim && k + VEC <= K) {
                        v[b] = *reinterpret_cast<const u32x4_elem<T>*>(src);
                        continue;
                    }
#pragma unroll
                    for (int j = 0; j < VEC; ++j) e[j] = (row < rlim && k + j < K) ? src[j] : T(0);
                } else {              // row = k, elements along mn
                    const int k = k0 + row, mn = c * VEC;
                    const T* src = panel + (int64_t)k * ld + mn;
                    if (ALIGNED && k < K && mn + VEC <= rlim) {
                        v[b] = *reinterpret_cast<const u32x4_elem<T>*>(src);
                        continue;
                    }
#pragma unroll
                    for (int j = 0; j < VEC; ++j) e[j] = (k < K && mn + j < rlim) ? src[j] : T(0);
                }
                v[b] = pack_chunk<T>(e);
            }
#pragma unroll
            for (int b = 0; b < GB; ++b) {
                const int q = tid + (i0 + b) * Cfg::THREADS;
                if ((CHUNKS % Cfg::THREADS != 0 || GL % GB != 0) && (i0 + b >= GL || q >= CHUNKS)) break;
                *reinterpret_cast<u32x4*>(lds + L::off(q / SCPR, q % SCPR + half * SCPR)) = v[b];
            }
            // keep the next batch's loads behind this batch's stores
            asm volatile("" ::: "memory");
        }
    }

    // ---- fragment reads (FragAddr: per-lane base registers + constants)
    using FA = FragAddr<Cfg, R, KC, KD, WT, NWP>;
    static constexpr int NREAD_PER_FRAG = FA::NPC;
    uint32_t fbase[FA::NBASE];

    __device__ __forceinline__ void init_frags(int lane, int wmn0)
    {
        static_for<FA::NBASE>([&](auto b_c) __attribute__((always_inline)) {
            constexpr int b = decltype(b_c)::value;
            fbase[b] = (uint32_t)(FA::off_of(FA::PLAN.base_combo[b], lane, wmn0) +
                                  FA::PLAN.base_shift[b]);
        });
    }
    // Make the bases opaque to the optimizer at the top of each K-step: every
    // read address is then formed inside the step as base + constant (the
    // constant goes into the instruction), instead of one register per
    // (stage, fragment, piece) hoisted out of the loop.
    __device__ __forceinline__ void refresh()
    {
        static_for<FA::NBASE>([&](auto b_c) __attribute__((always_inline)) {
            asm volatile("" : "+v"(fbase[decltype(b_c)::value]));
        });
    }
    template <int I, int KK, int PC>
    __device__ __forceinline__ const char* piece_addr(const char* buf) const
    {
        constexpr int x = FA::combo(I, KK, PC);
        return buf + fbase[FA::PLAN.cls[x]] + FA::PLAN.delta[x];
    }
    // piece PC of fragment (I, KK): 16 bytes (k-contiguous), 8 bytes (bf16
    // transposing read) or 4 bytes (fp32)
    template <int I, int KK, int PC>
    __device__ __forceinline__ u32x4 piece16(const char* buf) const
    {
        return *reinterpret_cast<const u32x4*>(piece_addr<I, KK, PC>(buf));
    }
    template <int I, int KK, int PC>
    __device__ __forceinline__ uint64_t piece8(const char* buf) const
    {
        typedef short s4 __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (__attribute__((address_space(3))) s4*)(
                                                    piece_addr<I, KK, PC>(buf))));
    }
    template <int I, int KK, int PC>
    __device__ __forceinline__ uint32_t piece4(const char* buf) const
    {
        return *reinterpret_cast<const uint32_t*>(piece_addr<I, KK, PC>(buf));
    }
    // the whole fragment (I, KK)
    template <int I, int KK>
    __device__ __forceinline__ u32x4 frag(const char* buf) const
    {
        if constexpr (KC) {
            return piece16<I, KK, 0>(buf);
        } else if constexpr (Cfg::ES == 4) {
            return u32x4{piece4<I, KK, 0>(buf), piece4<I, KK, 1>(buf), piece4<I, KK, 2>(buf),
                         piece4<I, KK, 3>(buf)};
        } else {
            const uint64_t lo = piece8<I, KK, 0>(buf), hi = piece8<I, KK, 1>(buf);
            return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
        }
    }
};

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt fields at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(n) lgkmcnt(0), expcnt untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// OUT_T: the kernel computes E = op(A) op(B) for a caller whose D is E
// transposed (D = op(B)^T op(A)^T with the operands passed swapped): the
// MFMA operands go in unswapped, so each lane's accumulator group holds four
// consecutive rows of E at one column, i.e. four adjacent columns of one row
// of D, and the epilogue still writes 16-byte vectors.
//
// OUT_BF16: C and D are bfloat16; alpha*acc + beta*C is formed in fp32 and
// rounded once to bf16 (round to nearest even, v_cvt_pk_bf16_f32).
//
// EPI: the fused epilogue of "GEMM on NVIDIA GPUs" (section 4, epilogue):
// after alpha*acc + beta*C, add the bias of the D column, apply the
// activation and the clamp, then convert and store -- all in registers, so
// no second kernel reads D back.
template <class Cfg, bool A_KC, bool B_KC, bool ALIGNED, bool SK = false, bool OUT_T = false,
          bool OUT_BF16 = false, bool EPI = false>
__global__ __launch_bounds__(Cfg::THREADS) __attribute__((amdgpu_waves_per_eu(Cfg::WPE)))
void dma_gemm_kernel(GemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, S = Cfg::S;
    constexpr int MF = Cfg::MF, NF = Cfg::NF, NKS = Cfg::NKS;
    using Acc = typename AccType<Cfg::KIND>::type;
    // Paired operands (see PAIR_) live in NP pair buffers and the others in
    // the S stage arrays (A's part first in either).
    constexpr bool PA = Cfg::pairs(A_KC, B_KC), PB = Cfg::pairs(B_KC, A_KC);
    constexpr bool PAIRED = PA || PB;
    constexpr int NP = Cfg::NP;
    using OpA = DmaOperand<Cfg, BM, A_KC, ALIGNED, PA, Cfg::WTM, Cfg::WM>;
    using OpB = DmaOperand<Cfg, BN, B_KC, ALIGNED, PB, Cfg::WTN, Cfg::WN>;
    constexpr int A_ST = PA ? 0 : OpA::BYTES, ST_BYTES = A_ST + (PB ? 0 : OpB::BYTES);
    constexpr int A_PR = PA ? OpA::BYTES : 0, PR_BYTES = A_PR + (PB ? OpB::BYTES : 0);
    constexpr int ST_DECL = ST_BYTES > 0 ? ST_BYTES : 16, PR_DECL = PR_BYTES > 0 ? PR_BYTES : 16;

    __shared__ __attribute__((aligned(1024))) char st0[ST_DECL];
    __shared__ __attribute__((aligned(1024))) char st1[ST_DECL];
    __shared__ __attribute__((aligned(1024))) char st2[ST_DECL];
    __shared__ __attribute__((aligned(1024))) char st3[S > 3 ? ST_DECL : 16];
    __shared__ __attribute__((aligned(1024))) char st4[S > 4 ? ST_DECL : 16];
    __shared__ __attribute__((aligned(1024))) char pr0[PR_DECL];
    __shared__ __attribute__((aligned(1024))) char pr1[PR_DECL];
    __shared__ __attribute__((aligned(1024))) char pr2[NP > 2 ? PR_DECL : 16];
    auto stage = [&](int s) __attribute__((always_inline)) -> char* {
        return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : s == 3 ? st3 : st4;
    };
    auto pr = [&](int i) __attribute__((always_inline)) -> char* {
        return i == 0 ? pr0 : i == 1 ? pr1 : pr2;
    };
    // Slots: the step in slot `cur` (its index mod P in a round of P steps)
    // has its staged operands in stage cur mod S and its paired ones in half
    // cur mod 2 of pair buffer cur/2 mod NP, i.e. at fragment steps shifted
    // by NKS in the second half.
    constexpr auto lcm = [](int x, int y) constexpr {
        int a = x, b = y;
        while (b != 0) {
            const int r = a % b;
            a = b;
            b = r;
        }
        return x / a * y;
    };
    // no staged operand with both paired: the stage ring plays no part
    constexpr int P = !PAIRED ? S : (PA && PB) ? 2 * NP : lcm(S, 2 * NP);
    static_assert(P % S == 0 || (PA && PB), "a round covers whole stage rings");
    static_assert(!PAIRED || P % (2 * NP) == 0, "a round covers whole pair-buffer cycles");
    static_assert(P <= 6, "slots of a round");
    auto a_lds = [&](int cur) __attribute__((always_inline)) -> char* {
        return PA ? pr((cur >> 1) % NP) : stage(cur % S);
    };
    auto b_lds = [&](int cur) __attribute__((always_inline)) -> char* {
        return PB ? pr((cur >> 1) % NP) + A_PR : stage(cur % S) + A_ST;
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wave_n0 = (wave % Cfg::WN) * Cfg::WTN;
    using T = typename Cfg::T;
    const T* A = static_cast<const T*>(p.A);
    const T* B = static_cast<const T*>(p.B);

    OpA oa;
    OpB ob;
    oa.init(wave, lane, p.lda);
    ob.init(wave, lane, p.ldb);
    oa.init_frags(lane, wave_m0);
    ob.init_frags(lane, wave_n0);
    // end of each stored matrix: A is M x K (k-contiguous) or K x M, B likewise
    const char* end_a = reinterpret_cast<const char*>(
        A + (A_KC ? (int64_t)(p.M - 1) * p.lda + p.K : (int64_t)(p.K - 1) * p.lda + p.M));
    const char* end_b = reinterpret_cast<const char*>(
        B + (B_KC ? (int64_t)(p.N - 1) * p.ldb + p.K : (int64_t)(p.K - 1) * p.ldb + p.N));
    const int nk_all = (p.K + BK - 1) / BK;  // K-steps of a whole tile
    const bool k_ragged = (p.K % BK) != 0;

    Acc acc[MF][NF];
    u32x4 fa[2][MF], fb[2][NF];

    // Copies in flight, per wave.  The barrier of step j issues the staged
    // operands' copy of step j + AHEAD (NST instructions), and with PAIR, on
    // odd j, the paired operands' copy of steps j + 2NP - 1 and j + 2NP
    // (NPR) into the pair buffer that step j finished.  Before
    // the barrier of step t the data of step t+1 must have landed: the count
    // of copy instructions issued after it, up to the barrier of step
    // `last`, may still be in flight (copies complete in issue order).
    constexpr int NST = (PA ? 0 : OpA::ND) + (PB ? 0 : OpB::ND);
    constexpr int NPR = (PA ? OpA::ND : 0) + (PB ? OpB::ND : 0);
    constexpr int AHEAD = Cfg::AHEAD;
    constexpr auto pair_in_flight = [](int t, int last) constexpr {
        // positions (step, 0 = staged / 1 = paired) of step t+1's copies
        const int js = t + 1 - AHEAD, jp = 2 * ((t + 1) >> 1) - 2 * NP + 1;
        int need = NPR > 0 ? 2 * jp + 1 : -1000;
        if (NST > 0 && 2 * js > need) need = 2 * js;
        int n = 0;
        for (int pos = need + 1; pos <= 2 * last + 1; ++pos) {
            const int j = pos >> 1;   // floor for negative positions too
            if ((pos & 1) == 0) n += NST;
            else if ((j & 1) != 0) n += NPR;
        }
        return n;
    };
    constexpr int WAIT_E = PAIRED ? pair_in_flight(12, 11) : Cfg::DMA_PER_STAGE * (AHEAD - 2);
    constexpr int WAIT_O = PAIRED ? pair_in_flight(13, 12) : Cfg::DMA_PER_STAGE * (AHEAD - 2);
    constexpr int WAIT_PRO = PAIRED ? pair_in_flight(-1, -1) : Cfg::DMA_PER_STAGE * (AHEAD - 1);
    static_assert(WAIT_E < 64 && WAIT_O < 64 && WAIT_PRO < 64, "vmcnt range");
    // The counts hold once every copy issued up to the barrier of step t-1
    // exists: steps up to t + LOOK.
    constexpr int LOOK = PAIRED ? (AHEAD - 1 > 2 * NP - 2 ? AHEAD - 1 : 2 * NP - 2) : AHEAD - 1;

    // The K-steps [k_lo, k_hi) of output tile (tm, tn), accumulated into acc
    // from zero.  Every wave enters with the LDS stages free.
    auto tile_work = [&](int tm, int tn, int k_lo, int k_hi) __attribute__((always_inline)) {
    const int m0 = tm * BM, n0 = tn * BN;
    const int rlim_a = p.M - m0, rlim_b = p.N - n0;
    const bool edge = rlim_a < BM || rlim_b < BN;
    const T* panel_a = A_KC ? A + (int64_t)m0 * p.lda : A + m0;
    const T* panel_b = B_KC ? B + (int64_t)n0 * p.ldb : B + n0;
    const i32x4 rsrc_a = OpA::panel_rsrc(panel_a, end_a);
    const i32x4 rsrc_b = OpB::panel_rsrc(panel_b, end_b);
    const int nk = k_hi - k_lo;              // steps of this range; step kt is K-step k_lo + kt
    const bool last = k_hi == nk_all;
    // Steps copied by DMA.  Rows past the matrix read as zero through the
    // buffer range and chunks that run past a row's end only feed outputs the
    // epilogue masks, so edge tiles use DMA too, except on their last step: a
    // chunk that straddles the end of the matrix would lose its last valid
    // bf16 element to the word-granular range check.  A ragged last step needs
    // exact zeros past K and is always register-staged.
    const int nk_dma = ALIGNED ? ((last && (k_ragged || edge)) ? nk - 1 : nk) : 0;

    // step kt of the staged operands into a stage array
    auto load = [&](int kt, char* base) __attribute__((always_inline)) {
        const int k0 = (k_lo + kt) * BK;
        if (kt < nk_dma) {
            if constexpr (!PA) oa.dma(rsrc_a, OpA::step_bytes(k0, p.lda), base, wave);
            if constexpr (!PB) ob.dma(rsrc_b, OpB::step_bytes(k0, p.ldb), base + A_ST, wave);
        } else {
            if constexpr (!PA) oa.guarded(panel_a, p.lda, rlim_a, k0, p.K, base, tid);
            if constexpr (!PB) ob.guarded(panel_b, p.ldb, rlim_b, k0, p.K, base + A_ST, tid);
        }
    };
    // steps 2q and 2q+1 of the paired operands into a pair buffer (one DMA
    // copy when both are DMA steps, else each existing step register-staged)
    auto load_pair = [&](int q, char* base) __attribute__((always_inline)) {
        const int k0 = (k_lo + 2 * q) * BK;
        if (2 * q + 1 < nk_dma) {
            if constexpr (PA) oa.dma(rsrc_a, OpA::step_bytes(k0, p.lda), base, wave);
            if constexpr (PB) ob.dma(rsrc_b, OpB::step_bytes(k0, p.ldb), base + A_PR, wave);
        } else {
#pragma unroll 1
            for (int h = 0; h < 2 && 2 * q + h < nk; ++h) {
                if constexpr (PA) oa.guarded(panel_a, p.lda, rlim_a, k0 + h * BK, p.K, base, tid, h);
                if constexpr (PB)
                    ob.guarded(panel_b, p.ldb, rlim_b, k0 + h * BK, p.K, base + A_PR, tid, h);
            }
        }
    };

#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = Acc{};

    // prologue: the copies the barriers of steps -VP .. -1 would have issued
    // (steps 0 .. AHEAD-1, and when paired pairs 0 .. NP-1), then wait for
    // step 0
    if constexpr (!PAIRED) {
#pragma unroll
        for (int s = 0; s < AHEAD; ++s)
            if (s < nk) load(s, stage(s));
        if (nk >= AHEAD) wait_vm_lgkm0<WAIT_PRO>();
        else wait_vm_lgkm0<0>();
    } else {
        constexpr int VP = AHEAD > 2 * NP - 1 ? AHEAD : 2 * NP - 1;
        static_for<VP>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int j = decltype(i_c)::value - VP;
            if constexpr (j + AHEAD >= 0)
                if (j + AHEAD < nk) load(j + AHEAD, stage((j + AHEAD) % S));
            if constexpr ((j & 1) != 0 && j + 2 * NP - 1 >= 0) {
                constexpr int q = (j + 2 * NP - 1) / 2;
                if (2 * q < nk) load_pair(q, pr(q % NP));
            }
        });
        if (nk > LOOK) wait_vm_lgkm0<WAIT_PRO>();
        else wait_vm_lgkm0<0>();
    }
    barrier_only();

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;

    // every fragment of fragment step KS of the step in slot CUR into fa/fb[BUF]
    auto read_frags = [&](auto cur_c, auto ks_c, auto buf_c) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value, KS = decltype(ks_c)::value;
        constexpr int BUF = decltype(buf_c)::value;
        constexpr int KA = KS + (PA ? (CUR & 1) * NKS : 0), KB = KS + (PB ? (CUR & 1) * NKS : 0);
        static_for<MF>([&](auto i_c) __attribute__((always_inline)) {
            fa[BUF][decltype(i_c)::value] = oa.template frag<decltype(i_c)::value, KA>(a_lds(CUR));
        });
        static_for<NF>([&](auto j_c) __attribute__((always_inline)) {
            fb[BUF][decltype(j_c)::value] = ob.template frag<decltype(j_c)::value, KB>(b_lds(CUR));
        });
    };
    read_frags(I0{}, I0{}, I0{});

    // Fragment step of a K-step at which the barrier sits, and the stage the
    // copy issued after it fills (relative to the current stage).
    constexpr int BAR_KS = Cfg::LATE ? NKS - 1 : NKS / 2;
    constexpr int FILL = Cfg::LATE ? 0 : S - 1;

    // One K-step held in slot CUR (static, so every LDS address is a
    // compile-time offset from its own __shared__ array), with run-time
    // checks: copies only for steps that exist, guarded copies allowed.
    auto step = [&](auto cur_c, int kt) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        constexpr int NXT = (CUR + 1) % P;
        constexpr int FAR = (CUR + FILL) % S;
        constexpr int WAIT = (CUR & 1) ? WAIT_O : WAIT_E;
        oa.refresh();
        ob.refresh();
        static_for<NKS>([&](auto ks_c) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_c)::value;
            if constexpr (ks == BAR_KS) {
                // the next step must have landed in every wave's part of LDS
                // (and, with the late barrier, this wave's reads of the stage
                // about to be refilled must be complete: lgkmcnt(0))
                if (kt + LOOK < nk) wait_vm_lgkm0<WAIT>();
                else wait_vm_lgkm0<0>();
                barrier_only();
                if (kt + AHEAD < nk) load(kt + AHEAD, stage(FAR));
                if constexpr (PAIRED && (CUR & 1) != 0)
                    if (kt + 2 * NP - 1 < nk) load_pair((kt + 2 * NP - 1) / 2, pr((CUR >> 1) % NP));
            }
            constexpr int cb = ks & 1;
            using NB = std::integral_constant<int, cb ^ 1>;
            if constexpr (ks + 1 < NKS) read_frags(cur_c, std::integral_constant<int, ks + 1>{}, NB{});
            else if (kt + 1 < nk) read_frags(std::integral_constant<int, NXT>{}, I0{}, NB{});
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j) {
                    if constexpr (OUT_T) mfma_step<Cfg::KIND>(fa[cb][i], fb[cb][j], acc[i][j]);
                    else mfma_step<Cfg::KIND>(fb[cb][j], fa[cb][i], acc[i][j]);
                }
        });
    };
    // Steady-state step with a pinned instruction order: every MFMA of a
    // fragment step is followed by one or two memory instructions (the next
    // fragment set's LDS reads and, in the second half, the DMA copies of the
    // step AHEAD ahead), so the matrix core is fed while loads are in flight.
    constexpr int RA = OpA::NREAD_PER_FRAG, RB = OpB::NREAD_PER_FRAG;
    constexpr int NREAD = MF * RA + NF * RB;
    constexpr int NMFMA = MF * NF;
    // the N-th of the NREAD memory instructions reading fragment step KS of
    // the step in slot CUR into fa/fb[BUF]
    auto read_op = [&](auto n_c, auto cur_c, auto ks_c, auto buf_c) __attribute__((always_inline)) {
        constexpr int N = decltype(n_c)::value, CUR = decltype(cur_c)::value;
        constexpr int KS = decltype(ks_c)::value, BUF = decltype(buf_c)::value;
        if constexpr (N < MF * RA) {
            constexpr int i = N / RA, pc = N % RA;
            constexpr int kk = KS + (PA ? (CUR & 1) * NKS : 0);
            const char* ab = a_lds(CUR);
            if constexpr (RA == 1) {
                fa[BUF][i] = oa.template piece16<i, kk, 0>(ab);
            } else if constexpr (RA == 4) {
                fa[BUF][i][pc] = oa.template piece4<i, kk, pc>(ab);
            } else {
                const uint64_t v = oa.template piece8<i, kk, pc>(ab);
                fa[BUF][i][2 * pc] = (uint32_t)v;
                fa[BUF][i][2 * pc + 1] = (uint32_t)(v >> 32);
            }
        } else {
            constexpr int m = N - MF * RA, j = m / RB, pc = m % RB;
            constexpr int kk = KS + (PB ? (CUR & 1) * NKS : 0);
            const char* bb = b_lds(CUR);
            if constexpr (RB == 1) {
                fb[BUF][j] = ob.template piece16<j, kk, 0>(bb);
            } else if constexpr (RB == 4) {
                fb[BUF][j][pc] = ob.template piece4<j, kk, pc>(bb);
            } else {
                const uint64_t v = ob.template piece8<j, kk, pc>(bb);
                fb[BUF][j][2 * pc] = (uint32_t)v;
                fb[BUF][j][2 * pc + 1] = (uint32_t)(v >> 32);
            }
        }
    };
    auto steady = [&](auto cur_c, int kt) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        constexpr int NXT = (CUR + 1) % P;
        constexpr int FAR = (CUR + FILL) % S;
        constexpr int WAIT = (CUR & 1) ? WAIT_O : WAIT_E;
        // copies issued at this step's barrier: the staged operands' step
        // AHEAD ahead, then (PAIR, odd slots) the paired operands' pair
        // starting 2NP - 1 steps ahead
        constexpr int NA_ST = PA ? 0 : OpA::ND, NB_ST = PB ? 0 : OpB::ND;
        constexpr int NA_PR = PA ? OpA::ND : 0;
        constexpr int NDMA = NST + ((PAIRED && (CUR & 1) != 0) ? NPR : 0);
        const int kst = (k_lo + kt + AHEAD) * BK, kpr = (k_lo + kt + 2 * NP - 1) * BK;
        const uint32_t ka = OpA::step_bytes(PA ? kpr : kst, p.lda);
        const uint32_t kb = OpB::step_bytes(PB ? kpr : kst, p.ldb);
        oa.refresh();
        ob.refresh();
        static_for<NKS>([&](auto ks_c) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_c)::value;
            constexpr int cb = ks & 1;
            constexpr bool mid = ks == BAR_KS;
            if constexpr (mid) {
                if constexpr (Cfg::LATE) wait_vm_lgkm0<WAIT>();
                else wait_vm<WAIT>();
                barrier_only();
            }
            constexpr int rcur = ks + 1 < NKS ? CUR : NXT;
            constexpr int rks = ks + 1 < NKS ? ks + 1 : 0;
            constexpr int nops = NREAD + (mid ? NDMA : 0);
            static_for<NMFMA>([&](auto e_c) __attribute__((always_inline)) {
                constexpr int e = decltype(e_c)::value;
                if constexpr (OUT_T)
                    mfma_step<Cfg::KIND>(fa[cb][e / NF], fb[cb][e % NF], acc[e / NF][e % NF]);
                else
                    mfma_step<Cfg::KIND>(fb[cb][e % NF], fa[cb][e / NF], acc[e / NF][e % NF]);
                __builtin_amdgcn_sched_barrier(0);
                // front-load: fragment reads go out over the first half of the
                // MFMAs (two per MFMA), DMA copies over the rest
                constexpr int HALF = NMFMA / 2;
                constexpr int lo = e < HALF ? e * NREAD / HALF
                                            : NREAD + (e - HALF) * (nops - NREAD) / (NMFMA - HALF);
                constexpr int hi = e + 1 < HALF ? (e + 1) * NREAD / HALF
                                 : e + 1 == HALF ? NREAD
                                                 : NREAD + (e + 1 - HALF) * (nops - NREAD) / (NMFMA - HALF);
                static_for<hi - lo>([&](auto oo_c) __attribute__((always_inline)) {
                    constexpr int o = lo + decltype(oo_c)::value;
                    constexpr int d = o - NREAD;
                    if constexpr (o < NREAD)
                        read_op(std::integral_constant<int, o>{}, std::integral_constant<int, rcur>{},
                                std::integral_constant<int, rks>{},
                                std::integral_constant<int, cb ^ 1>{});
                    else if constexpr (d < NA_ST)
                        oa.dma_one(d, rsrc_a, ka, stage(FAR), wave);
                    else if constexpr (d < NA_ST + NB_ST)
                        ob.dma_one(d - NA_ST, rsrc_b, kb, stage(FAR) + A_ST, wave);
                    else if constexpr (d < NA_ST + NB_ST + NA_PR)
                        oa.dma_one(d - NA_ST - NB_ST, rsrc_a, ka, pr((CUR >> 1) % NP), wave);
                    else
                        ob.dma_one(d - NA_ST - NB_ST - NA_PR, rsrc_b, kb, pr((CUR >> 1) % NP) + A_PR,
                                   wave);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    int kt = 0;
    // steady state: every step of the round issues its copies as DMA (the
    // last step of a round copies up to step kt + P - 1 + LAST_AHEAD)
    constexpr int LAST_AHEAD = PAIRED && AHEAD < 2 * NP ? 2 * NP : AHEAD;
    for (; kt + P - 1 + LAST_AHEAD < nk_dma; kt += P) {
        steady(I0{}, kt);
        steady(I1{}, kt + 1);
        if constexpr (P > 2) steady(I2{}, kt + 2);
        if constexpr (P > 3) steady(I3{}, kt + 3);
        if constexpr (P > 4) steady(I4{}, kt + 4);
        if constexpr (P > 5) steady(I5{}, kt + 5);
    }
    // tail: remaining steps with run-time checks (guarded copies allowed)
    for (; kt < nk; kt += P) {
        step(I0{}, kt);
        if (kt + 1 < nk) step(I1{}, kt + 1);
        if constexpr (P > 2)
            if (kt + 2 < nk) step(I2{}, kt + 2);
        if constexpr (P > 3)
            if (kt + 3 < nk) step(I3{}, kt + 3);
        if constexpr (P > 4)
            if (kt + 4 < nk) step(I4{}, kt + 4);
        if constexpr (P > 5)
            if (kt + 5 < nk) step(I5{}, kt + 5);
    }
    };  // tile_work

    // Index (in f32x4 units) of a thread's accumulator group (i, j, vg) in a
    // stream-K partial-sum slot: consecutive threads hold consecutive 16 bytes.
    constexpr int TILE_F = BM * BN;
    auto part_index = [&](int i, int j, int vg) __attribute__((always_inline)) {
        return ((i * NF + j) * (Cfg::ACC / 4) + vg) * Cfg::THREADS + tid;
    };
    // Partial-sum slot of workgroup c as a buffer, accessed at device scope
    // (cache policy SC1): stores are written through to where every XCD sees
    // them and loads do not return lines another XCD's L2 may hold stale, so
    // the hand-off needs no whole-cache write-back or invalidate.
    constexpr int CPOL_SC1 = 16;
    auto part_rsrc = [&](int64_t c) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc(p.sk_partials + c * TILE_F, 0, TILE_F * 4,
                                                 0x00020000);
    };

    // C and D element type, and 4-element vector access to them.  D is
    // written once and not read back by this kernel, so its stores are
    // non-temporal: streamed out without displacing the operand panels that
    // other workgroups are still reading (8192x14336x4096 bf16: 0.769 ->
    // 0.715 ms on MI355X).  C loads stay ordinary: non-temporal ones measured
    // slower (4096^3 with beta: 0.118 -> 0.127 ms).
    using OutT = std::conditional_t<OUT_BF16, bf16_t, float>;
    auto load4 = [](const OutT* q) __attribute__((always_inline)) -> f32x4 {
        if constexpr (OUT_BF16) {
            const u16x4 h = *reinterpret_cast<const u16x4_a2*>(q);
            return f32x4{to_f32(h[0]), to_f32(h[1]), to_f32(h[2]), to_f32(h[3])};
        } else {
            return *reinterpret_cast<const f32x4_a4*>(q);
        }
    };
    auto store4 = [](OutT* q, f32x4 v) __attribute__((always_inline)) {
        if constexpr (OUT_BF16)
            __builtin_nontemporal_store(__builtin_convertvector(v, bf16x4),
                                        reinterpret_cast<bf16x4_a2*>(q));
        else
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_a4*>(q));
    };

    // ---- epilogue.  A lane's accumulator group holds 4 adjacent columns of
    // one D row, so direct stores would write each row 32 bytes per
    // instruction (every 128-byte line in four pieces, from four
    // instructions).  Instead each batch of FM D rows (fragment row i, or
    // fragment column j when the output is transposed) goes through LDS
    // (the stage arrays are free once the mainloop is done): the lanes write
    // their groups into a per-wave [FM][DC] fp32 block, 16-byte chunks
    // XOR-swizzled by row so neither the column-wise writes nor the row-wise
    // reads conflict, then read it back so that consecutive lanes hold
    // consecutive 16-byte pieces of one row.  beta*C loads and D stores then
    // cover whole rows of the wave's block per instruction ("GEMM on NVIDIA
    // GPUs", section 4: the epilogue stores the accumulator in the output
    // layout).  Stream-K partial sums (contributors c0..c1, none when
    // c0 == c1) are added in registers, in workgroup order, before staging.
    // poison: write NaN-scaled results (a stream-K finisher whose wait for a
    // contributor gave up; the sticky error word is the authoritative signal)
    auto epilogue = [&](int tm, int tn, int64_t c0, int64_t c1, bool poison = false)
                        __attribute__((always_inline)) {
    const int m0 = tm * BM, n0 = tn * BN;
    const float alpha = poison ? __builtin_nanf("") : p.alpha, beta = p.beta;
    constexpr int VG = Cfg::ACC / 4;
    // D is M x N, or N x M when the output is transposed
    const int d_rows = OUT_T ? p.N : p.M, d_cols = OUT_T ? p.M : p.N;
    const int in_frag = FM == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4);
    constexpr int NO = OUT_T ? NF : MF, NQA = OUT_T ? MF : NF;
    // the blocks use the first NSA stage arrays, or the pair buffers when
    // those are larger (naming only those keeps the others out of the kernel
    // when S does not need them)
    constexpr bool USE_PR = PR_BYTES > ST_BYTES;
    constexpr int ARR = USE_PR ? PR_BYTES : ST_BYTES;
    constexpr int MAXA = USE_PR ? 2 : (S < 3 ? S : 3);
    // fragment columns staged per pass: all NQA of a fragment row when every
    // wave's block fits in MAXA arrays and a staged row divides a 64-lane
    // read, else half of them in two passes, else one per pass (three
    // fragment columns: 24 chunks per row would not divide the read)
    constexpr auto fits = [](int qb) constexpr {
        const int ch = qb * FM / 4;
        const int wps = ARR / (FM * qb * FM * 4);
        return ch >= 8 && ch <= 64 && 64 % ch == 0 && wps >= 1 &&
               (Cfg::WAVES + wps - 1) / wps <= MAXA;
    };
    constexpr int NQ = fits(NQA) ? NQA : (NQA % 2 == 0 && fits(NQA / 2)) ? NQA / 2 : 1;
    static_assert(NQ >= 1 && NQA % NQ == 0 && fits(NQ), "staging space");
    constexpr int QH = NQA / NQ;       // passes per fragment row
    constexpr int DC = NQ * FM;        // D columns of the wave's block in one pass
    constexpr int CH = DC / 4;         // 16-byte chunks per staged row
    constexpr int RPI = 64 / CH;       // staged rows per read instruction
    constexpr int NT = FM / RPI;       // read instructions per batch
    constexpr int REGION = FM * DC * 4;
    constexpr int WPS = ARR / REGION;  // wave blocks per array
    static_assert(64 % CH == 0, "staging shape");
    // row r's chunks are XORed with r mod 16 (mod CH for narrower rows)
    constexpr int SWZ = CH >= 16 ? 15 : CH - 1;
    constexpr int NSA = (Cfg::WAVES + WPS - 1) / WPS;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    char* base = USE_PR ? pr0 : st0;
    if constexpr (NSA > 1) base = wv / WPS == 1 ? (USE_PR ? pr1 : st1) : base;
    if constexpr (NSA > 2) base = wv / WPS == 2 ? st2 : base;
    char* const region = base + (wv % WPS) * REGION;
    auto slot = [&](int r, int chunk) __attribute__((always_inline)) -> f32x4* {
        return reinterpret_cast<f32x4*>(region + r * (DC * 4) + ((chunk ^ (r & SWZ)) * 16));
    };
    // first D row and column of the wave's block; the lane's 4 D columns in
    // pass qh start at col0 + qh * DC
    const int wr0 = OUT_T ? n0 + wave_n0 : m0 + wave_m0;
    const int col0 = (OUT_T ? m0 + wave_m0 : n0 + wave_n0) + 4 * (lane % CH);
    // whole tile inside D with 16-byte rows: no per-row or per-element checks
    const bool interior = m0 + BM <= p.M && n0 + BN <= p.N && p.d_vec &&
                          (beta == 0.0f || p.c_vec);
    // the lane's columns are the same in every fragment row: their bias is
    // read once
    float bias4[QH][4] = {};
    if constexpr (EPI) {
#pragma unroll
        for (int qh = 0; qh < QH; ++qh)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (col0 + qh * DC + s < d_cols) bias4[qh][s] = bias_of<OutT>(p, col0 + qh * DC + s);
    }
    __syncthreads();  // every wave is done reading operands from the stage arrays
    static_for<NO * QH>([&](auto oq_c) __attribute__((always_inline)) {
        constexpr int o = decltype(oq_c)::value / QH, qh = decltype(oq_c)::value % QH;
        const int col = col0 + qh * DC;
        const bool col_vec = p.d_vec && col + 4 <= d_cols;
        f32x4 sum[NQ][VG];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int i = OUT_T ? qh * NQ + q : o, j = OUT_T ? o : qh * NQ + q;
#pragma unroll
            for (int vg = 0; vg < VG; ++vg)
                sum[q][vg] = f32x4{acc[i][j][4 * vg], acc[i][j][4 * vg + 1], acc[i][j][4 * vg + 2],
                                   acc[i][j][4 * vg + 3]};
        }
        if constexpr (SK) {
            for (int64_t c = c0; c < c1; ++c) {
                const auto rsrc = part_rsrc(c);
                f32x4 v[NQ][VG];
#pragma unroll
                for (int q = 0; q < NQ; ++q)
#pragma unroll
                    for (int vg = 0; vg < VG; ++vg)
                        v[q][vg] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rsrc,
                                       part_index(OUT_T ? qh * NQ + q : o, OUT_T ? o : qh * NQ + q, vg) * 16,
                                       0, CPOL_SC1));
#pragma unroll
                for (int q = 0; q < NQ; ++q)
#pragma unroll
                    for (int vg = 0; vg < VG; ++vg) sum[q][vg] += v[q][vg];
            }
        }
        // stage: the lane's row lane % FM, columns q*FM + 8*vg + in_frag
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int vg = 0; vg < VG; ++vg)
                *slot(lane % FM, (q * FM + 8 * vg + in_frag) / 4) = sum[q][vg];
        // read back row-wise: lane holds chunk lane % CH of rows t*RPI + lane / CH.
        // Runtime loops keep this code small: the epilogue runs once per tile
        // from instruction memory, and every copy of an unrolled body is
        // fetched again for each tile.
        const int row0 = wr0 + o * FM + lane / CH;
        // interior tiles: the activation and the clamp are compile-time
        // choices of the loop, so its body has no branches
        // The C rows of a group of CG read instructions are loaded before any
        // of the group's D rows is stored, so CG loads are in flight per lane
        // (the compiler cannot move a C load above an earlier D store itself:
        // C and D may be the same matrix).  Every element is still read
        // before it is written, so C == D stays correct.
        constexpr int CG = NT < 4 ? NT : 4;
        auto interior_rows = [&](auto act_c, auto clamp_c) __attribute__((always_inline)) {
#pragma unroll 1
            for (int t0 = 0; t0 < NT; t0 += CG) {
                f32x4 cv[CG];
                if (beta != 0.0f) {
#pragma unroll
                    for (int u = 0; u < CG; ++u)
                        cv[u] = load4(reinterpret_cast<const OutT*>(p.C) +
                                      (int64_t)(row0 + (t0 + u) * RPI) * p.ldc + col);
                }
#pragma unroll
                for (int u = 0; u < CG; ++u) {
                    const int t = t0 + u;
                    const int64_t row = row0 + t * RPI;
                    f32x4 out = alpha * *slot(t * RPI + lane / CH, lane % CH);
                    if (beta != 0.0f) out += beta * cv[u];
                    if constexpr (EPI)
                        out = epilogue_fixed4<decltype(act_c)::value, decltype(clamp_c)::value>(
                            p, out, bias4[qh]);
                    store4(reinterpret_cast<OutT*>(p.D) + row * p.ldd + col, out);
                }
            }
        };
        using A0 = std::integral_constant<int, EPI_ACT_NONE>;
        using A1 = std::integral_constant<int, EPI_ACT_RELU>;
        using A2 = std::integral_constant<int, EPI_ACT_GELU>;
        using C0 = std::false_type;
        using C1 = std::true_type;
        if (interior) {
            if constexpr (EPI) {
                if (p.act == EPI_ACT_RELU) {
                    if (p.clamp) interior_rows(A1{}, C1{}); else interior_rows(A1{}, C0{});
                } else if (p.act == EPI_ACT_GELU) {
                    if (p.clamp) interior_rows(A2{}, C1{}); else interior_rows(A2{}, C0{});
                } else {
                    if (p.clamp) interior_rows(A0{}, C1{}); else interior_rows(A0{}, C0{});
                }
            } else {
                interior_rows(A0{}, C0{});
            }
        } else {
            // edge tiles: rows past D skipped, columns masked; C rows of a
            // group loaded ahead of its stores as on interior tiles
#pragma unroll 1
            for (int t0 = 0; t0 < NT; t0 += CG) {
                f32x4 cv[CG];
                if (beta != 0.0f) {
#pragma unroll
                    for (int u = 0; u < CG; ++u) {
                        const int row = row0 + (t0 + u) * RPI;
                        cv[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        if (row >= d_rows) continue;
                        const OutT* crow = reinterpret_cast<const OutT*>(p.C) + (int64_t)row * p.ldc;
                        if (p.c_vec && col + 4 <= d_cols) {
                            cv[u] = load4(crow + col);
                        } else {
#pragma unroll
                            for (int s = 0; s < 4; ++s)
                                if (col + s < d_cols) cv[u][s] = to_f32(crow[col + s]);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < CG; ++u) {
                    const int t = t0 + u;
                    const int row = row0 + t * RPI;
                    if (row >= d_rows) continue;
                    f32x4 out = alpha * *slot(t * RPI + lane / CH, lane % CH);
                    if (beta != 0.0f) out += beta * cv[u];
                    if constexpr (EPI) out = epilogue_op4(p, out, bias4[qh]);
                    OutT* drow = reinterpret_cast<OutT*>(p.D) + (int64_t)row * p.ldd;
                    if (col_vec) {
                        store4(drow + col, out);
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            if (col + s < d_cols) drow[col + s] = from_f32<OutT>(out[s]);
                    }
                }
            }
        }
    });
    };  // epilogue

    if constexpr (!SK) {
        int tm, tn;
        tile_coords(p, tm, tn);
        tile_work(tm, tn, 0, nk_all);
        epilogue(tm, tn, 0, 0);
    } else {
        // Stream-K ("GEMM on NVIDIA GPUs", section 5: split-K partial sums
        // P^(s) = sum over a K range, reduced afterwards).  The grid's G
        // workgroups split the W = tiles * nk_all (tile, K-step) iterations
        // evenly (sk_ranges.hpp).  A tile is finished by the workgroup that
        // reaches its last K-step; every other workgroup touching the tile
        // ends its range inside it, stores its partial sums to its own
        // workspace slot and raises its flag (a workgroup contributes to at
        // most one tile: the one its range ends in).  A workgroup does that
        // contributing segment first and its whole tiles next, so no
        // contribution waits behind another tile's fix-up; the finishing
        // segment comes last.  The finisher waits for the lower-numbered
        // contributors, adds their partials in workgroup (= K) order, so the
        // result is reproducible, clears their flags and runs the epilogue.
        // Contributions are published before any wait, and a finisher only
        // waits for lower-numbered workgroups, which the host keeps resident
        // at the same time (the grid never exceeds the workgroup slots), so
        // the waits cannot deadlock.  They are bounded as well (p.sk_spin
        // polls per contributor): a finisher that gives up adds no partial
        // and clears no flag, writes NaN to its tile and sets the sticky
        // error word; the host reports it and clears the whole flag area.
        __shared__ int sk_ok;
        const int64_t W = (int64_t)p.tiles_m * p.tiles_n * nk_all;
        const int64_t G = gridDim.x, g = blockIdx.x;
        const SkRange rg = sk_range(W, G, g, nk_all);
        const int64_t w_end = rg.w_end;
        // one segment: the iterations from w to the end of w's tile or of the
        // range, whichever comes first
        auto segment = [&](int64_t w) __attribute__((always_inline)) {
            const int t = (int)(w / nk_all);
            const int k_lo = (int)(w - (int64_t)t * nk_all);
            const int64_t t_end = (int64_t)(t + 1) * nk_all;
            const int k_hi = (int)((w_end < t_end ? w_end : t_end) - (int64_t)t * nk_all);
            int tm, tn;
            tile_of(p, t, tm, tn);
            __syncthreads();  // the previous segment's reads of the LDS stages are done
            tile_work(tm, tn, k_lo, k_hi);
            if (k_hi == nk_all) {
                // contributors: the workgroups owning iterations t*nk_all .. w-1
                const int64_t c0 = k_lo > 0 ? sk_owner((int64_t)t * nk_all, W, G) : g;
                bool ok = true;
                if (c0 < g) {
                    if (tid == 0) {
                        int got = 1;
                        for (int64_t c = c0; c < g && got; ++c) {
                            got = 0;
                            for (int it = 0; it < p.sk_spin; ++it) {
                                if (__hip_atomic_load(p.sk_flags + c, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                                    got = 1;
                                    break;
                                }
                                __builtin_amdgcn_s_sleep(2);
                            }
                        }
                        if (got) {
                            for (int64_t c = c0; c < g; ++c)
                                __hip_atomic_store(p.sk_flags + c, 0u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        } else {
                            __hip_atomic_store(p.sk_error, 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        }
                        sk_ok = got;
                    }
                    __syncthreads();
                    ok = sk_ok != 0;
                }
                if (ok) epilogue(tm, tn, c0, g);
                else epilogue(tm, tn, g, g, true);
            } else {
                const auto rsrc = part_rsrc(g);
#pragma unroll
                for (int i = 0; i < MF; ++i)
#pragma unroll
                    for (int j = 0; j < NF; ++j)
#pragma unroll
                        for (int vg = 0; vg < Cfg::ACC / 4; ++vg)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(u32x4, f32x4{acc[i][j][4 * vg], acc[i][j][4 * vg + 1],
                                                                acc[i][j][4 * vg + 2],
                                                                acc[i][j][4 * vg + 3]}),
                                rsrc, part_index(i, j, vg) * 16, 0, CPOL_SC1);
                wait_vm<0>();     // every partial store has been acknowledged
                __syncthreads();  // ... in every wave
                if (tid == 0)
                    __hip_atomic_store(p.sk_flags + g, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        // The host keeps every range within two tiles' worth of iterations,
        // so a range is at most a first tile's tail (or the whole first
        // tile), one whole tile, and a last tile's head: three straight-line
        // segments (a loop over them keeps far more registers live).
        if (rg.w0 >= w_end) return;
        if (rg.head) segment(rg.t_last * nk_all);
        if (rg.mid) segment((rg.t_first + 1) * nk_all);
        segment(rg.w0);
    }
}

}  // namespace dg
