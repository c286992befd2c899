// gemm_kernel.h -- the tiled int8 MFMA GEMM with the fused LLM.int8() epilogue.
//
// C[t,n] = sum_k Xq[t,k] * CB[n,k] accumulates exactly in int32 (LLM.int8()
// summary, kurtkim.github.io, section "Int8 Matrix Multiplication with 16-bit
// Float Inputs and Outputs").  The epilogue dequantizes by the outer product
// of the row and column scales, a[t] * SCB[n] / 127^2 (section "Vector-wise
// Quantization"), adds the fp16 product of the outlier columns of X with the
// matching dequantized weight rows and the bias, and rounds once to fp16
// (section "The Core of LLM.int8(): Mixed-precision Decomposition"; the
// agentlenshq.com write-up, "Core idea" step 3).
//
// Design (gfx950):
//  * Block tile BM x BN, ROWB (64 or 128) bytes of K per pipeline stage,
//    STAGES stages in LDS filled by direct global->LDS 16-byte loads (no
//    VGPR staging): each wavefront load instruction fills 1 KB = 1024/ROWB
//    staged rows.
//  * Both operands are K-contiguous ([T,K] and [N,K]), so A and B fragments
//    have the same shape: a lane reads 16 consecutive bytes of one row.  The
//    16-byte chunks of staged row r are XOR-swizzled (chunk c in slot
//    c ^ swz(r)) so the 16-byte fragment reads of consecutive rows spread
//    over all LDS banks.
//  * Wavefronts are WM x WN over the block tile, each owning FM x FN
//    accumulator tiles of 32x32 (v_mfma_i32_32x32x32_i8; the k order inside
//    an MFMA is irrelevant for an exact integer sum because A and B use the
//    same lane -> k mapping).
//  * The fp16 outlier product, with v_mfma_f32_32x32x16_f16 accumulating
//    onto the dequantized fp32 values: up to 32 outlier columns as two MFMAs
//    per accumulator tile in k_gemm's epilogue; more in k_gemm_many, which
//    runs it as a second pass through the same pipeline over the gathered
//    fp16 operands (K' = n padded to a multiple of 64).
//  * Tiles are numbered XCD-aware: workgroup ids are dealt round-robin over
//    the 8 XCDs, so each XCD gets a contiguous run of tile ids, and tile ids
//    walk a grouped raster (GROUP tile rows at a time) for L2 reuse.
#pragma once

#include <type_traits>
#include <utility>

#include "internal.h"

namespace llmint8 {
namespace gemm {
namespace {   // internal linkage: nothing here is exported from the library

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;

template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int GROUP_, int ROWB_ = 64>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, GROUP = GROUP_;
    static constexpr int ROWB = ROWB_;                  // bytes of each operand row per stage
    static constexpr int kKSteps = ROWB / 32;           // 32-deep MFMA k-steps per stage
    static constexpr int kChunks = ROWB / 16;           // 16-byte chunks per staged row
    static constexpr int kRowsPerInstr = 1024 / ROWB;   // rows one 1 KB load instruction fills
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
    static constexpr int kAInstr = BM / kRowsPerInstr / kWaves;   // load instructions per wave per stage
    static constexpr int kBInstr = BN / kRowsPerInstr / kWaves;
    static constexpr int kLoads = kAInstr + kBInstr;
    static constexpr int kStageBytes = (BM + BN) * ROWB;
    static constexpr int kLdsBytes = STAGES * kStageBytes;
    static_assert(ROWB == 64 || ROWB == 128, "stage depth");
    static_assert(BM % (kRowsPerInstr * kWaves) == 0 && BN % (kRowsPerInstr * kWaves) == 0,
                  "load split");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
    static_assert(STAGES >= 2, "pipeline depth");
    static_assert((STAGES - 1) * kLoads < 64, "vmcnt range");

    // Slot swizzle of staged row r, measured on gfx950: 16-lane groups of
    // ds_read_b128 cover all 64 banks.  64-byte rows put rows r, r+4, r+8,
    // r+12 on the same banks, 128-byte rows put every other row there.
    __device__ __forceinline__ static int swz(int r)
    {
        return ROWB == 64 ? (r >> 2) & 3 : (r >> 1) & 7;
    }
};

// One 16-byte direct global->LDS load per lane through a buffer resource:
// the lane's 16 bytes at voffset + soffset land at LDS dst + 16 * lane (dst
// wave-uniform, passed in M0).  A plain function rather than inline builtin
// calls in the templates below, so that the host compilation pass, which
// has no such builtin, only ever sees this one declaration.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, lds_void *dst,
                                           uint32_t voffset, uint32_t soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voffset, soffset, 0, 0);
}

// One 16-byte load per lane into registers through a buffer resource (lane
// offset voffset, wave-uniform soffset); a plain function for the same
// reason as lds_load16.
__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                          uint32_t soffset)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0));
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void tile_coords(int bid, int nblk, int ntm, int ntn, int group, int &tm,
                                            int &tn)
{
    const int q = nblk / kXcds, r = nblk % kXcds;
    const int x = bid % kXcds, loc = bid / kXcds;
    const int t = x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
    const int per_group = group * ntn;
    const int g = t / per_group, first = g * group;
    const int gs = ntm - first < group ? ntm - first : group;
    const int w = t - g * per_group;
    tm = first + w % gs;
    tn = w / gs;
}

// One operand pair streamed through the LDS ring.  Each operand is read
// through a buffer resource based at the tile's first row, so a load
// instruction takes a constant per-lane 32-bit offset (row * ld + swizzled
// chunk, fixed for the whole loop) plus the stage's k byte as a scalar
// offset, and its LDS destination in M0: no per-load address arithmetic.
template <class C>
struct Streams {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t offA[C::kAInstr], offB[C::kBInstr];

    // Buffer over [base, base + bytes): raw (stride 0) 32-bit words; the
    // extent is capped at 4 GB - 1 (every offset used stays below it).
    __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const char *base, int64_t bytes)
    {
        const uint32_t n = bytes > 0xffffffffll ? 0xffffffffu : (uint32_t)bytes;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, (int)n,
                                                 0x00020000);
    }

    __device__ __forceinline__ void init(const char *abase, int64_t lda, int64_t m0, int64_t mrows,
                                         const char *bbase, int64_t ldb, int64_t n0, int64_t nrows,
                                         int wave, int lane)
    {
        ra = rsrc(abase + m0 * lda, (mrows - m0) * lda);
        rb = rsrc(bbase + n0 * ldb, (nrows - n0) * ldb);
        // lane l fills LDS bytes [16l, 16l+16) of its instruction's KB: row
        // l / kChunks, slot l % kChunks, which holds chunk slot ^ swz(row)
        const int lr = lane / C::kChunks, ls = lane % C::kChunks;
#pragma unroll
        for (int j = 0; j < C::kAInstr; ++j) {
            const int r = (wave * C::kAInstr + j) * C::kRowsPerInstr + lr;
            const int64_t row = m0 + r < mrows ? r : mrows - 1 - m0;   // ragged: clamp
            offA[j] = (uint32_t)(row * lda + ((ls ^ C::swz(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < C::kBInstr; ++j) {
            const int r = (wave * C::kBInstr + j) * C::kRowsPerInstr + lr;
            const int64_t row = n0 + r < nrows ? r : nrows - 1 - n0;
            offB[j] = (uint32_t)(row * ldb + ((ls ^ C::swz(r)) << 4));
        }
    }

    // The j-th of this wave's kLoads load instructions for a stage (A first).
    __device__ __forceinline__ void issue_one(char *smem, int stage, int64_t kbyte, int wave,
                                              int j) const
    {
        char *sa = smem + stage * C::kStageBytes;
        char *sb = sa + C::BM * C::ROWB;
        if (j < C::kAInstr)
            lds_load16(ra, (lds_void *)(sa + (wave * C::kAInstr + j) * 1024), offA[j],
                       (uint32_t)kbyte);
        else
            lds_load16(rb, (lds_void *)(sb + (wave * C::kBInstr + j - C::kAInstr) * 1024),
                       offB[j - C::kAInstr], (uint32_t)kbyte);
    }

    __device__ __forceinline__ void issue(char *smem, int stage, int64_t kbyte, int wave) const
    {
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j)
            issue_one(smem, stage, kbyte, wave, j);
    }

    // The A operand's loads only (the fp16 pass stages its B operand itself).
    __device__ __forceinline__ void issue_a(char *smem, int stage, int64_t kbyte, int wave) const
    {
#pragma unroll
        for (int j = 0; j < C::kAInstr; ++j)
            issue_one(smem, stage, kbyte, wave, j);
    }
};

struct MfmaI8 {
    typedef v16i acc_t;
    __device__ __forceinline__ static acc_t op(v4i a, v4i b, acc_t c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

// fp16 MFMA on accumulators that hold fp32 bit patterns in the same
// registers as the int32 sums (the epilogue converts them in place).
struct MfmaF16 {
    typedef v16i acc_t;
    __device__ __forceinline__ static acc_t op(v4i a, v4i b, acc_t c)
    {
        return __builtin_bit_cast(
            v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                         __builtin_bit_cast(v8h, b),
                                                         __builtin_bit_cast(v16f, c), 0, 0, 0));
    }
};

// fp16 MFMA on fp32 accumulators (the many-outlier pass).
struct MfmaF16F {
    typedef v16f acc_t;
    __device__ __forceinline__ static acc_t op(v4i a, v4i b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                      __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    }
};

// Fragments of one 32-deep k-step: FM A-fragments and FN B-fragments.
template <class C>
struct Frags {
    v4i a[C::FM], b[C::FN];
};

template <class C>
__device__ __forceinline__ void read_frags(Frags<C> &f, const char *sa, const char *sb, int fo)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
        f.a[i] = *reinterpret_cast<const v4i *>(sa + i * 32 * C::ROWB + fo);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        f.b[j] = *reinterpret_cast<const v4i *>(sb + j * 32 * C::ROWB + fo);
}

template <class C, class M>
__device__ __forceinline__ void mfmas(const Frags<C> &f, typename M::acc_t (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = M::op(f.a[i], f.b[j], acc[i][j]);
}

// The g-th fragment read of a k-step, in the order the MFMAs (row-major over
// (i, j)) first need them: a0, b0 .. b(FN-1), a1 .. a(FM-1).  The last read
// then has FN*(FM-1) MFMAs of the next k-step to land.
template <class C>
__device__ __forceinline__ void read_one(Frags<C> &f, const char *sa, const char *sb, int fo, int g)
{
    if (g == 0)
        f.a[0] = *reinterpret_cast<const v4i *>(sa + fo);
    else if (g <= C::FN)
        f.b[g - 1] = *reinterpret_cast<const v4i *>(sb + (g - 1) * 32 * C::ROWB + fo);
    else
        f.a[g - C::FN] = *reinterpret_cast<const v4i *>(sa + (g - C::FN) * 32 * C::ROWB + fo);
}

// One k-step in a fixed issue order: groups of (one global->LDS load, one
// fragment read of a later k-step, FM*FN/groups MFMAs of this k-step),
// pinned with scheduling barriers so the loads and reads always sit between
// MFMAs and the matrix core never waits on their issue.  Loads kL0 ..
// kL0+kNL-1 of the stage being refilled are issued here.
template <class C, class M, int kL0, int kNL>
__device__ __forceinline__ void kstep(const Frags<C> &cur, Frags<C> &nxt, const char *sa,
                                      const char *sb, int fo,
                                      typename M::acc_t (&acc)[C::FM][C::FN],
                                      const Streams<C> &st, char *smem, int stage, int64_t kbyte,
                                      int wave)
{
    constexpr int kReads = C::FM + C::FN, kMfma = C::FM * C::FN;
    constexpr int kGroups = kReads > kNL ? kReads : kNL;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        if (g < kNL)
            st.issue_one(smem, stage, kbyte, wave, kL0 + g);
        if (g < kReads)
            read_one<C>(nxt, sa, sb, fo, g);
#pragma unroll
        for (int idx = g * kMfma / kGroups; idx < (g + 1) * kMfma / kGroups; ++idx) {
            const int i = idx / C::FN, j = idx % C::FN;
            acc[i][j] = M::op(cur.b[j], cur.a[i], acc[i][j]);   // D[n][t]: see k_gemm
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <class C, class M, bool kWithLoads>
__device__ __forceinline__ void half_stage(const Frags<C> &cur, Frags<C> &nxt, const char *sa,
                                           const char *sb, int fo,
                                           typename M::acc_t (&acc)[C::FM][C::FN],
                                           const Streams<C> &st, char *smem, int stage,
                                           int64_t kbyte, int wave)
{
    kstep<C, M, 0, kWithLoads ? C::kLoads : 0>(cur, nxt, sa, sb, fo, acc, st, smem, stage, kbyte,
                                                wave);
}

// s_waitcnt lgkmcnt(0) with vmcnt/expcnt left alone: every LDS read issued
// by this wavefront has returned.
__device__ __forceinline__ void wait_lds()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// The main loop for 128-byte stages (4 k-steps): fragments are read two
// k-steps ahead (three fragment buffers), so every wavefront is done
// reading a stage after its second k-step; the barrier sits there, and the
// refill of the stage's buffer (stage kt+STAGES) is spread over its last two
// k-steps instead of being issued in one burst, which had stalled the MFMA
// stream behind the load issue.  Buffer use, waits and tail handling as in
// mainloop; the fragment buffers rotate with period 3 stages (12 k-steps),
// so the loop body is three stages long and 1 or 2 leftover stages run after
// it.
template <class C, class M>
__device__ __forceinline__ void mainloop_ra2(char *smem, const Streams<C> &st, int numK,
                                             typename M::acc_t (&acc)[C::FM][C::FN], int wm,
                                             int wn, int wave, int lane)
{
    static_assert(C::kKSteps == 4 && C::kLoads % 2 == 0, "128-byte stages");
    const int frow = (lane & 31) * C::ROWB;
    int fo[C::kKSteps];
#pragma unroll
    for (int s = 0; s < C::kKSteps; ++s)
        fo[s] = frow + (((2 * s + (lane >> 5)) ^ C::swz(lane & 31)) << 4);
    const int aoff = wm * (C::BM / C::WM) * C::ROWB;
    const int boff = C::BM * C::ROWB + wn * (C::BN / C::WN) * C::ROWB;
    const int64_t klast = (int64_t)(numK - 1) * C::ROWB;
    auto kb = [&](int s) -> int64_t {
        const int64_t k = (int64_t)s * C::ROWB;
        return k < klast ? k : klast;
    };
    auto stage_a = [&](int s) { return smem + (s % C::STAGES) * C::kStageBytes + aoff; };
    auto stage_b = [&](int s) { return smem + (s % C::STAGES) * C::kStageBytes + boff; };

#pragma unroll
    for (int s = 0; s < C::STAGES; ++s)
        st.issue(smem, s, kb(s), wave);
    wait_vm<(C::STAGES - 1) * C::kLoads>();   // stage 0 landed
    __builtin_amdgcn_s_barrier();

    Frags<C> F[3];
    read_frags<C>(F[0], stage_a(0), stage_b(0), fo[0]);
    read_frags<C>(F[1], stage_a(0), stage_b(0), fo[1]);
    constexpr int kHalf = C::kLoads / 2;
    // stage kt whose k-step 0 uses fragment buffer P (kt % 3 == P mod 3 in
    // the unrolled period): k-step s uses F[(4P + s) % 3] and reads k-step
    // s+2 into F[(4P + s + 2) % 3]
    auto stage = [&]<int P>(std::integral_constant<int, P>, int kt) {
        const int nk = kt + 1 < numK ? kt + 1 : kt;
        const int rb = kt % C::STAGES;
        const int64_t kr = kb(kt + C::STAGES);
        kstep<C, M, 0, 0>(F[(4 * P) % 3], F[(4 * P + 2) % 3], stage_a(kt), stage_b(kt), fo[2], acc,
                          st, smem, 0, 0, wave);
        kstep<C, M, 0, 0>(F[(4 * P + 1) % 3], F[(4 * P + 3) % 3], stage_a(kt), stage_b(kt), fo[3],
                          acc, st, smem, 0, 0, wave);
        // every read of stage kt has been issued; once they have returned and
        // stage kt+1 has landed, the wavefronts meet and stage kt's buffer is
        // refilled over the next two k-steps
        wait_lds();
        wait_vm<(C::STAGES - 2) * C::kLoads>();
        __builtin_amdgcn_s_barrier();
        kstep<C, M, 0, kHalf>(F[(4 * P + 2) % 3], F[(4 * P + 4) % 3], stage_a(nk), stage_b(nk),
                              fo[0], acc, st, smem, rb, kr, wave);
        kstep<C, M, kHalf, kHalf>(F[(4 * P + 3) % 3], F[(4 * P + 5) % 3], stage_a(nk),
                                  stage_b(nk), fo[1], acc, st, smem, rb, kr, wave);
    };
    int kt = 0;
    for (; kt + 3 <= numK; kt += 3) {
        stage(std::integral_constant<int, 0>{}, kt);
        stage(std::integral_constant<int, 1>{}, kt + 1);
        stage(std::integral_constant<int, 2>{}, kt + 2);
    }
    if (numK - kt >= 1)
        stage(std::integral_constant<int, 0>{}, kt);
    if (numK - kt >= 2)
        stage(std::integral_constant<int, 1>{}, kt + 1);
    wait_vm<0>();   // the tail loads land before anyone reuses the buffers
}

// Runs numK stages (ROWB bytes of K = ROWB/32 32-deep k-steps each) of the
// pipelined main loop.  Stage s is loaded into LDS buffer s % STAGES.  A
// buffer is free once every wavefront has read its stage's last k-step,
// which the barrier before the stage's last k-step of MFMAs establishes; the
// stage STAGES ahead is issued into it right there, so all STAGES buffers
// are busy and a stage's loads have STAGES-1 trips to land.  Every trip
// loads exactly one stage (stages past the end reload the last one into a
// buffer nobody reads again), so the number of loads in flight at each wait
// is a constant and the loop body has no branches for the scheduler to stop
// at.  The barrier sits before the last k-step of a stage, so the MFMAs
// issued before it keep the matrix cores busy while the wavefronts meet.
// Fragments of the next k-step are read from LDS under the current one's
// MFMAs.
template <class C, class M>
__device__ __forceinline__ void mainloop(char *smem, const Streams<C> &st, int numK,
                                         typename M::acc_t (&acc)[C::FM][C::FN], int wm, int wn,
                                         int wave, int lane)
{
    // fragment read offsets: row (lane&31) of each 32-row tile, chunk
    // 2s + lane/32 for k-step s of the stage
    const int frow = (lane & 31) * C::ROWB;
    int fo[C::kKSteps];
#pragma unroll
    for (int s = 0; s < C::kKSteps; ++s)
        fo[s] = frow + (((2 * s + (lane >> 5)) ^ C::swz(lane & 31)) << 4);
    const int aoff = wm * (C::BM / C::WM) * C::ROWB;
    const int boff = C::BM * C::ROWB + wn * (C::BN / C::WN) * C::ROWB;
    const int64_t klast = (int64_t)(numK - 1) * C::ROWB;
    auto kb = [&](int s) -> int64_t {
        const int64_t k = (int64_t)s * C::ROWB;
        return k < klast ? k : klast;
    };
    auto stage_a = [&](int s) { return smem + (s % C::STAGES) * C::kStageBytes + aoff; };
    auto stage_b = [&](int s) { return smem + (s % C::STAGES) * C::kStageBytes + boff; };

#pragma unroll
    for (int s = 0; s < C::STAGES; ++s)
        st.issue(smem, s, kb(s), wave);
    wait_vm<(C::STAGES - 1) * C::kLoads>();   // stage 0 landed
    __builtin_amdgcn_s_barrier();

    Frags<C> f0, f1;
    read_frags<C>(f0, stage_a(0), stage_b(0), fo[0]);
    for (int kt = 0; kt < numK; ++kt) {
#pragma unroll
        for (int s = 0; s < C::kKSteps; ++s) {
            Frags<C> &cur = s % 2 == 0 ? f0 : f1;
            Frags<C> &nxt = s % 2 == 0 ? f1 : f0;
            if (s + 1 < C::kKSteps) {
                // reads of k-step s+1 under the MFMAs of k-step s
                half_stage<C, M, false>(cur, nxt, stage_a(kt), stage_b(kt), fo[s + 1], acc, st,
                                        smem, 0, 0, wave);
            } else {
                wait_vm<(C::STAGES - 2) * C::kLoads>();   // stage kt+1 landed
                __builtin_amdgcn_s_barrier();
                // every wavefront has read all of stage kt: refill its buffer
                // with stage kt+STAGES, and read the next stage's k-step 0,
                // under the last k-step's MFMAs
                const int nk = kt + 1 < numK ? kt + 1 : kt;
                half_stage<C, M, true>(cur, nxt, stage_a(nk), stage_b(nk), fo[0], acc, st, smem,
                                       kt % C::STAGES, kb(kt + C::STAGES), wave);
            }
        }
    }
    wait_vm<0>();   // the tail loads land before anyone reuses the buffers
}

// FP8 variant: v_mfma_f32_32x32x64_f8f6f4 on FP8 codes (the instruction's
// format 0 is E4M3, 1 is E5M2; the same for both operands, no block scales)
// with fp32 accumulators.  A 64-deep k-step
// takes 32 bytes per lane: lane half h reads 16-byte chunks 4s + h and
// 4s + 2 + h of the 64-byte k-step s, for A and B alike, so both operands
// hold the same k values in the same places and the sum covers all 64.
template <int kFmt>
struct MfmaF8 {
    typedef v16f acc_t;
    static constexpr int kCode = kFmt == kF8E4M3 ? 0 : 1;
    __device__ __forceinline__ static acc_t op(v8i a, v8i b, acc_t c)
    {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kCode, kCode, 0, 0, 0, 0);
    }
};

template <class C>
struct Frags8 {
    v8i a[C::FM], b[C::FN];
};

__device__ __forceinline__ v8i frag8(const char *p, int fo0, int fo1)
{
    const v4i lo = *reinterpret_cast<const v4i *>(p + fo0);
    const v4i hi = *reinterpret_cast<const v4i *>(p + fo1);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// read_one's order (a0, b0 .. b(FN-1), a1 .. a(FM-1)) for 32-byte fragments.
template <class C>
__device__ __forceinline__ void read_one8(Frags8<C> &f, const char *sa, const char *sb, int fo0,
                                          int fo1, int g)
{
    if (g == 0)
        f.a[0] = frag8(sa, fo0, fo1);
    else if (g <= C::FN)
        f.b[g - 1] = frag8(sb + (g - 1) * 32 * C::ROWB, fo0, fo1);
    else
        f.a[g - C::FN] = frag8(sa + (g - C::FN) * 32 * C::ROWB, fo0, fo1);
}

// kstep for the FP8 k-steps: the same groups of (load issue, fragment read,
// MFMAs) pinned by scheduling barriers.
template <class C, int kFmt, int kL0, int kNL>
__device__ __forceinline__ void kstep8(const Frags8<C> &cur, Frags8<C> &nxt, const char *sa,
                                       const char *sb, int fo0, int fo1,
                                       v16f (&acc)[C::FM][C::FN], const Streams<C> &st,
                                       char *smem, int stage, int64_t kbyte, int wave)
{
    constexpr int kReads = C::FM + C::FN, kMfma = C::FM * C::FN;
    constexpr int kGroups = kReads > kNL ? kReads : kNL;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        if (g < kNL)
            st.issue_one(smem, stage, kbyte, wave, kL0 + g);
        if (g < kReads)
            read_one8<C>(nxt, sa, sb, fo0, fo1, g);
#pragma unroll
        for (int idx = g * kMfma / kGroups; idx < (g + 1) * kMfma / kGroups; ++idx) {
            const int i = idx / C::FN, j = idx % C::FN;
            acc[i][j] = MfmaF8<kFmt>::op(cur.b[j], cur.a[i], acc[i][j]);   // D[n][t], as k_gemm
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The pipelined main loop of `mainloop` (same stage ring, waits, barrier
// and refill placement) over ROWB/64 FP8 k-steps per stage (codes of
// format kFmt).
template <class C, int kFmt>
__device__ __forceinline__ void mainloop_f8(char *smem, const Streams<C> &st, int numK,
                                            v16f (&acc)[C::FM][C::FN], int wm, int wn, int wave,
                                            int lane)
{
    constexpr int kS = C::ROWB / 64;
    const int frow = (lane & 31) * C::ROWB, h = lane >> 5, sw = C::swz(lane & 31);
    int fo0[kS], fo1[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s) {
        fo0[s] = frow + (((4 * s + h) ^ sw) << 4);
        fo1[s] = frow + (((4 * s + 2 + h) ^ sw) << 4);
    }
    const int aoff = wm * (C::BM / C::WM) * C::ROWB;
    const int boff = C::BM * C::ROWB + wn * (C::BN / C::WN) * C::ROWB;
    const int64_t klast = (int64_t)(numK - 1) * C::ROWB;
    auto kb = [&](int s) -> int64_t {
        const int64_t k = (int64_t)s * C::ROWB;
        return k < klast ? k : klast;
    };
    auto stage_a = [&](int s) { return smem + (s % C::STAGES) * C::kStageBytes + aoff; };
    auto stage_b = [&](int s) { return smem + (s % C::STAGES) * C::kStageBytes + boff; };

#pragma unroll
    for (int s = 0; s < C::STAGES; ++s)
        st.issue(smem, s, kb(s), wave);
    wait_vm<(C::STAGES - 1) * C::kLoads>();   // stage 0 landed
    __builtin_amdgcn_s_barrier();

    Frags8<C> f0, f1;
#pragma unroll
    for (int g = 0; g < C::FM + C::FN; ++g)
        read_one8<C>(f0, stage_a(0), stage_b(0), fo0[0], fo1[0], g);
    for (int kt = 0; kt < numK; ++kt) {
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            Frags8<C> &cur = s % 2 == 0 ? f0 : f1;
            Frags8<C> &nxt = s % 2 == 0 ? f1 : f0;
            if (s + 1 < kS) {
                kstep8<C, kFmt, 0, 0>(cur, nxt, stage_a(kt), stage_b(kt), fo0[s + 1], fo1[s + 1], acc,
                                st, smem, 0, 0, wave);
            } else {
                wait_vm<(C::STAGES - 2) * C::kLoads>();   // stage kt+1 landed
                __builtin_amdgcn_s_barrier();
                const int nk = kt + 1 < numK ? kt + 1 : kt;
                kstep8<C, kFmt, 0, C::kLoads>(cur, nxt, stage_a(nk), stage_b(nk), fo0[0], fo1[0], acc,
                                        st, smem, kt % C::STAGES, kb(kt + C::STAGES), wave);
            }
        }
        // with an odd number of k-steps per stage the buffers swap roles
        if constexpr (kS % 2 == 1) {
            const Frags8<C> t = f0;
            f0 = f1;
            f1 = t;
        }
    }
    wait_vm<0>();   // the tail loads land before anyone reuses the buffers
}

// The main loop for the stage shape: read-two-ahead for the int8 product
// over 128-byte stages (the fp16 pass over many outlier columns keeps the
// one-ahead loop: its fp32 accumulators leave no room for the third
// fragment buffer).
template <class C, class M>
__device__ __forceinline__ void run_mainloop(char *smem, const Streams<C> &st, int numK,
                                             typename M::acc_t (&acc)[C::FM][C::FN], int wm,
                                             int wn, int wave, int lane)
{
    if constexpr (C::kKSteps == 4 && std::is_same_v<M, MfmaI8>)
        mainloop_ra2<C, M>(smem, st, numK, acc, wm, wn, wave, lane);
    else
        mainloop<C, M>(smem, st, numK, acc, wm, wn, wave, lane);
}

// The finished fp16 block tile is staged in LDS (BM rows of BN*2 bytes) and
// written out row by row in 16-byte pieces, so that every store instruction
// fills whole 128-byte lines; straight from the accumulator layout each
// store would touch 32 rows.  8-byte unit u of tile row r sits in slot
// u ^ (r % 32): the 32 rows of an accumulator tile write one unit each
// without bank conflicts, and a 16-byte read of units 2k, 2k+1 finds them in
// slot k ^ ((r % 32) / 2), halves swapped when r is odd.
template <class C>
__device__ __forceinline__ void write_tile(const char *smem, const EpilogueArgs &ep, int64_t m0,
                                           int64_t n0, int64_t T, int64_t N, int tid)
{
    constexpr int kPieces = C::BN / 8;                 // 16-byte pieces per tile row
    constexpr int kRowsPerPass = C::kThreads / kPieces;
    const int k = tid % kPieces;
#pragma unroll 4
    for (int r = tid / kPieces; r < C::BM; r += kRowsPerPass) {
        const int64_t t = m0 + r, n = n0 + 8 * k;
        uint4 v = *reinterpret_cast<const uint4 *>(smem + r * (C::BN * 2) +
                                                   16 * (k ^ ((r & 31) >> 1)));
        if (r & 1)
            v = make_uint4(v.z, v.w, v.x, v.y);
        if (t < T && n < N)
            *reinterpret_cast<uint4 *>(ep.out + t * N + n) = v;
    }
}

// The fp16 outlier operands of a tile (up to 32 outlier columns): the x_out
// rows of its BM rows and the w_out rows of its BN columns, 32 halves (64
// bytes) each, held in the LDS bytes after the ring (BM+BN rows; chunk q of
// row r in slot q ^ ((r >> 2) & 3), so that the 16 rows a quarter-wave reads
// cover all banks).  They do not depend on the GEMM: each wavefront issues a
// quarter of them as direct global->LDS loads before its first stage, so they
// have landed when the main loop starts and cost no registers during it.
template <class C>
struct OutlierRows {
    static constexpr int kRowBytes = 64;
    static constexpr int kBytes = (C::BM + C::BN) * kRowBytes;
    static constexpr int kInstr = kBytes / 1024 / C::kWaves;   // load instructions per wave
    static_assert(kBytes % (1024 * C::kWaves) == 0 && (C::BM / 16) % kInstr == 0,
                  "whole instructions, each within x or w rows");
    __device__ __forceinline__ static int slot(int r, int q) { return q ^ ((r >> 2) & 3); }
};

template <class C>
__device__ __forceinline__ void issue_outlier_rows(char *orows, const EpilogueArgs &ep,
                                                   int64_t m0, int64_t n0, int64_t T, int64_t N,
                                                   int wave, int lane)
{
    using R = OutlierRows<C>;
    const char *xb = reinterpret_cast<const char *>(ep.x_out);
    const char *wb = static_cast<const char *>(ep.w_out);
    // every row read lies inside the workspace's x_out / w_out segments (at
    // least 2*K >= 64 bytes per row); with n = 0 their contents are unused
    const __amdgpu_buffer_rsrc_t rx = Streams<C>::rsrc(xb + m0 * R::kRowBytes, (T - m0) * R::kRowBytes);
    const __amdgpu_buffer_rsrc_t rw = Streams<C>::rsrc(wb + n0 * R::kRowBytes, (N - n0) * R::kRowBytes);
    const int lr = lane / 4, lq = lane % 4;
#pragma unroll
    for (int u = 0; u < R::kInstr; ++u) {
        const int j = wave * R::kInstr + u;          // 16 staged rows per instruction
        const int r = 16 * j + lr;                   // staged row: x rows, then w rows
        const bool isx = 16 * j < C::BM;
        const int64_t rr = isx ? r : r - C::BM;      // row within the tile's rows / columns
        const int64_t lim = isx ? T - m0 : N - n0;
        const int64_t row = rr < lim ? rr : lim - 1;   // ragged: clamp
        const uint32_t off = (uint32_t)(row * R::kRowBytes + 16 * R::slot(r, lq));
        lds_load16(isx ? rx : rw, (lds_void *)(orows + j * 1024), off, 0);
    }
}

// 16 bytes of staged outlier row r: halves 8c .. 8c+7.
template <class C>
__device__ __forceinline__ v4i outlier_frag(const char *orows, int r, int c)
{
    return *reinterpret_cast<const v4i *>(orows + r * OutlierRows<C>::kRowBytes +
                                          16 * OutlierRows<C>::slot(r, c));
}

// Zero-point variant, per output row t: ia = 1/nd_a[t], za = zp_a[t] and
// ra = rs_a[t] + K*zp_a[t] (mod 2^32), so that the shifted integer sum of
// an output is C + zp_b[n]*ra + za*rs_b[n] -- exact in wrapping 32-bit
// arithmetic because its true value fits int32 (K <= 33286).
__device__ __forceinline__ void zp_row(const EpilogueArgs &ep, int64_t t, int64_t K, float &ia,
                                       int &za, int &ra)
{
    ia = zp_inv(ep.a[t]);
    const int2 z = ep.row_zp[t];
    za = z.x;
    ra = (int)((unsigned)z.y + (unsigned)K * (unsigned)z.x);
}

// Zero-point variant: the dequantized int8 part of one output, from the
// int8 sum acc, the row's za and ra, the column's zp_b and rs_b, and 1/nd_a
// (ia) and nd_b.
__device__ __forceinline__ float zp_dequant(int acc, int za, int ra, int zb, int rb, float ia,
                                            float ndb)
{
    const unsigned c = (unsigned)acc + (unsigned)zb * (unsigned)ra + (unsigned)za * (unsigned)rb;
    return (float)(int)c * (ia * zp_inv(ndb));
}

// Up to 32 outlier columns: their fp16 fragments (loaded before the main
// loop, rows of 32 halves) go straight into the MFMAs, and each 32x32
// accumulator tile is finished on its own (dequantize, fp16 MFMA over the
// outlier columns, bias, round) in a few VGPRs and staged in LDS, which every
// wavefront has stopped reading; then the whole block tile is written out.
// Operands come from clamped addresses and the column scales are loaded one
// column group ahead, so no latency is paid per accumulator tile.
template <class C, bool kBias, bool kRelu, bool kZp, class Acc = v16i>
__device__ __forceinline__ void finish_tile(const Acc (&acc)[C::FM][C::FN], const float (&at)[C::FM],
                                            const int (&za)[C::FM], const int (&ra)[C::FM],
                                            const char *orows,
                                            char *smem, const EpilogueArgs &ep, int64_t m0,
                                            int64_t n0, int64_t T, int64_t N, int nout, int wm,
                                            int wn, int lane, int tid)
{
    static_assert(C::BM * C::BN * 2 <= C::kLdsBytes, "output tile fits the LDS ring");
    const int tl = lane & 31, nl = 4 * (lane >> 5);
    const int64_t nw = n0 + wn * (C::BN / C::WN);
    // outlier fragments from LDS: lane (tl, hi) holds halves 8*(2*s2 + hi) ..
    // +7 of its row for the 16-deep k-step s2
    const int hi = lane >> 5;
    v4i xo[C::FM][2];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            xo[i][s2] = outlier_frag<C>(orows, wm * (C::BM / C::WM) + i * 32 + tl, 2 * s2 + hi);
    // column factors and bias of column group j, fetched one group ahead
    v4f sn[2][4];
    // zero-point variant: zp and code sums of the group's columns, loaded at
    // the start of their own group (double-buffering them too spills)
    v4i zb[4], rb[4];
    uint2 bias[2][4];
    auto load_cols = [&](int j, int buf) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int64_t nc = nw + j * 32 + 8 * g + nl;
            nc = nc < N ? nc : N - 4;
            sn[buf][g] = *reinterpret_cast<const v4f *>(ep.scb + nc);
            if constexpr (kBias)
                bias[buf][g] = *reinterpret_cast<const uint2 *>(ep.bias + nc);
        }
    };
    load_cols(0, 0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        if (j + 1 < C::FN)
            load_cols(j + 1, (j + 1) % 2);
        const int cb = j % 2;
        if constexpr (kZp) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                int64_t nc = nw + j * 32 + 8 * g + nl;
                nc = nc < N ? nc : N - 4;
                zb[g] = *reinterpret_cast<const v4i *>(ep.zp_b + nc);
                rb[g] = *reinterpret_cast<const v4i *>(ep.rs_b + nc);
            }
        }
        v4i wo[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            wo[s2] = outlier_frag<C>(orows, C::BM + wn * (C::BN / C::WN) + j * 32 + tl, 2 * s2 + hi);
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            v16f d;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (kZp)
                    d[r] = zp_dequant(acc[i][j][r], za[i], ra[i], zb[r / 4][r % 4],
                                      rb[r / 4][r % 4], at[i], sn[cb][r / 4][r % 4]);
                else
                    d[r] = (float)acc[i][j][r] * (at[i] * sn[cb][r / 4][r % 4]);
            }
            if (nout > 0) {
                d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, wo[0]),
                                                         __builtin_bit_cast(v8h, xo[i][0]), d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, wo[1]),
                                                         __builtin_bit_cast(v8h, xo[i][1]), d, 0, 0, 0);
            }
            // bias, one rounding, staged: registers 4g..4g+3 hold tile columns
            // nc + 8g .. nc + 8g + 3 of tile row tr
            const int tr = wm * (C::BM / C::WM) + i * 32 + tl;
            const int nc = wn * (C::BN / C::WN) + j * 32 + nl;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint16_t h[4];
                if constexpr (kBias) {
                    const uint2 bb = bias[cb][g];
                    const float bv[4] = {h2f((uint16_t)(bb.x & 0xffffu)), h2f((uint16_t)(bb.x >> 16)),
                                         h2f((uint16_t)(bb.y & 0xffffu)), h2f((uint16_t)(bb.y >> 16))};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        h[q] = f2h_act<kRelu>(d[4 * g + q] + bv[q]);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        h[q] = f2h_act<kRelu>(d[4 * g + q]);
                }
                const int u = (nc + 8 * g) / 4;
                *reinterpret_cast<uint2 *>(smem + tr * (C::BN * 2) + 8 * (u ^ (tr & 31))) =
                    make_uint2((unsigned)h[0] | ((unsigned)h[1] << 16),
                               (unsigned)h[2] | ((unsigned)h[3] << 16));
            }
        }
    }
    __syncthreads();
    write_tile<C>(smem, ep, m0, n0, T, N, tid);
}

// ---------------------------------------------------------------------------
// More than 32 outlier columns: the fp16 product as a second GEMM pass on the
// tile, onto the dequantized int8 result, in stages of 64 outlier positions
// (128 bytes of fp16 per operand row) through two LDS buffers.  Its operands
// depend on the mode the row quantization chose (see internal.h):
//   kOutCompact  A = x_out [T, ld] (fp16), B = the gathered weight codes
//                [N, ld] (int8); stage s = positions 64s .. 64s+63;
//   kOutDense    A = X [T, K], B = CB [N, K] themselves; stage s = the s-th
//                non-empty 64-column group, and B's codes of the group's
//                non-outlier columns are masked to zero (so A needs no mask).
// A is staged by direct global->LDS loads like the int8 operands.  B goes
// through registers: each lane loads 16 codes of a weight row, dequantizes
// them to fp16 -- fp16(cb * fp32(SCB/127)), the correctly rounded CB*SCB/127
// (dequant_w_r); zero-point and FP8 variants as their outlier weights -- and
// writes them into the stage in the layout the fragment reads expect.  The
// codes of stage s+2 are loaded while stage s is multiplied and written
// during stage s+1, so neither operand stalls the MFMAs for long.
// ---------------------------------------------------------------------------
template <class C>
using PassCfg = Cfg<C::BM, C::BN, C::WM, C::WN, 2, C::GROUP, 128>;

// Dequantization parameters of one weight row (output column): absmax s =
// fp32(SCB/127); FP8 s = the scale 2^-e; zero-point s = fp32(1/nd), zp, nd.
struct DqRow {
    float s;
    int zp;
    float nd;
};

// kVarF8: E5M2 codes, kVarF8E4: E4M3 codes.
enum { kVarAbsmax = 0, kVarZp = 1, kVarF8 = 2, kVarF8E4 = 3 };
constexpr int var_f8(int var)
{
    return var == kVarF8 ? kF8E5M2 : var == kVarF8E4 ? kF8E4M3 : kF8None;
}

template <int kVar>
__device__ __forceinline__ DqRow dq_row(const EpilogueArgs &ep, int64_t n)
{
    DqRow p{0.0f, 0, 0.0f};
    if constexpr (kVar == kVarZp) {
        p.nd = ep.scb[n];
        p.zp = ep.zp_b[n];
        p.s = p.nd > 0.0f ? 1.0f / p.nd : 0.0f;
    } else if constexpr (var_f8(kVar) != kF8None) {
        p.s = ep.scb[n];
    } else {
        p.s = ep.scb[n] / 127.0f;
    }
    return p;
}

// 8 weight codes (bytes of w0, w1) -> 8 fp16 values; code e is kept only when
// bit e of m8 is set (an outlier column), else 0.
template <int kVar>
__device__ __forceinline__ uint4 dq8(unsigned w0, unsigned w1, unsigned m8, const DqRow &p)
{
    unsigned h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const unsigned byte = ((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xffu;
        uint16_t v;
        if constexpr (var_f8(kVar) != kF8None)
            v = dequant_w_f8<var_f8(kVar)>(byte, p.s);
        else if constexpr (kVar == kVarZp)
            v = dequant_w_zp_r((int)(int8_t)byte, p.zp, p.nd, p.s);
        else
            v = dequant_w_r((int)(int8_t)byte, p.s);
        h[e] = ((m8 >> e) & 1u) ? v : 0u;
    }
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

// 4 weight codes (bytes of w) -> 4 fp16 values, masked like dq8.
template <int kVar>
__device__ __forceinline__ uint2 dq4(unsigned w, unsigned m4, const DqRow &p)
{
    unsigned h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const unsigned byte = (w >> (8 * e)) & 0xffu;
        uint16_t v;
        if constexpr (var_f8(kVar) != kF8None)
            v = dequant_w_f8<var_f8(kVar)>(byte, p.s);
        else if constexpr (kVar == kVarZp)
            v = dequant_w_zp_r((int)(int8_t)byte, p.zp, p.nd, p.s);
        else
            v = dequant_w_r((int)(int8_t)byte, p.s);
        h[e] = ((m4 >> e) & 1u) ? v : 0u;
    }
    return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

// The byte mask of 4 codes from their 4 outlier flags (bit e -> byte e).
__device__ __forceinline__ unsigned byte_mask4(unsigned m4)
{
    return ((m4 * 0x00204081u) & 0x01010101u) * 0xffu;
}

// dq4 for the variants whose code 0 dequantizes to +0 (absmax, FP8): the
// codes of non-outlier columns are cleared first (bytemask), so the masking
// costs one instruction per 4 codes, and the halves are built in place
// (v_fma_mixlo / v_fma_mixhi: one instruction per value after the int8
// conversion).
template <int kVar>
__device__ __forceinline__ uint2 dq4m(unsigned w, unsigned bytemask, const DqRow &p)
{
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    w &= bytemask;
    h2v h[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const unsigned byte = (w >> (8 * e)) & 0xffu;
        float v;
        if constexpr (var_f8(kVar) != kF8None)
            v = f8_to_f<var_f8(kVar)>(byte) * p.s;
        else
            v = (float)(int)(int8_t)byte * p.s;
        h[e / 2][e % 2] = (_Float16)v;
    }
    return make_uint2(__builtin_bit_cast(unsigned, h[0]), __builtin_bit_cast(unsigned, h[1]));
}

// The B operand of the pass: lane l loads 16 codes (positions 16 (l % 4) ..
// of the stage) of weight row wave * kRows + 16 i + l / 4 (rows past N read
// row N-1, never stored), dequantizes them with its row's parameters and
// writes them to the stage's B region as 2 fp16 chunks (2 (l % 4) and the
// next), in slot chunk ^ swz(row) like the direct-loaded operands.
template <class C, int kVar>
struct BStage {
    static constexpr int kRows = C::BN / C::kWaves;   // weight rows a wavefront stages
    static constexpr int kI = kRows / 16;              // 16-byte code loads per lane per stage
    static constexpr int kUnits = 4 * kI;              // 4-code conversion units per stage
    static_assert(kRows % 16 == 0, "16 rows x 4 pieces per load instruction");
    __amdgpu_buffer_rsrc_t tile;   // the tile's rows n0 .. N-1
    uint32_t off[kI];
    int row[kI], piece;
    DqRow prm[kI];
    v4i reg[2][kI];   // codes of two stages (by stage parity)

    __device__ __forceinline__ void init(const int8_t *base, int64_t ld, int64_t n0, int64_t N,
                                         const EpilogueArgs &ep, int wave, int lane)
    {
        tile = Streams<C>::rsrc(reinterpret_cast<const char *>(base + n0 * ld), (N - n0) * ld);
        piece = lane & 3;
#pragma unroll
        for (int i = 0; i < kI; ++i) {
            row[i] = wave * kRows + 16 * i + (lane >> 2);
            const int64_t r = n0 + row[i] < N ? row[i] : N - 1 - n0;
            off[i] = (uint32_t)(r * ld + 16 * piece);
            prm[i] = dq_row<kVar>(ep, n0 + r);
        }
    }

    template <int kBuf>
    __device__ __forceinline__ void load(int col)
    {
#pragma unroll
        for (int i = 0; i < kI; ++i)
            reg[kBuf][i] = buf_load16(tile, off[i], (uint32_t)col);
    }

    // Unit u of the stage in buffer kBuf: codes 4 (u % 4) .. of load u / 4,
    // i.e. half u % 2 of chunk 2 * piece + (u % 4) / 2; m16: bit e set =
    // position 16 * piece + e is an outlier column.
    // bm: the byte masks of the lane's 4 code words (byte_mask4 of m16's
    // nibbles), used by the variants whose code 0 is +0
    template <int kBuf>
    __device__ __forceinline__ void store_unit(char *stage, unsigned m16, const unsigned (&bm)[4],
                                               int u) const
    {
        const int i = u / 4, sub = u % 4;
        const int r = row[i];
        uint2 h;
        if constexpr (kVar == kVarZp)
            h = dq4<kVar>((unsigned)reg[kBuf][i][sub], (m16 >> (4 * sub)) & 0xfu, prm[i]);
        else
            h = dq4m<kVar>((unsigned)reg[kBuf][i][sub], bm[sub], prm[i]);
        char *sb = stage + C::BM * C::ROWB;
        *reinterpret_cast<uint2 *>(sb + r * C::ROWB + 16 * ((2 * piece + sub / 2) ^ C::swz(r)) +
                                   8 * (sub % 2)) = h;
    }
};

// One fp16 k-step of the pass: the fragment reads of the next k-step
// interleaved with this one's MFMAs, pinned in groups like kstep's.
// work(g) (a generic callable) runs between the g-th read and its MFMAs, so
// VALU work can be spread over the k-step.
template <class C, class AccArray, class Work>
__device__ __forceinline__ void pass_kstep(const Frags<C> &cur, Frags<C> &nxt, const char *sa,
                                           const char *sb, int fo, AccArray &acc, Work &&work)
{
    constexpr int kReads = C::FM + C::FN, kMfma = C::FM * C::FN;
#pragma unroll
    for (int g = 0; g < kReads; ++g) {
        read_one<C>(nxt, sa, sb, fo, g);
        work(std::integral_constant<int, 0>{}, g);
#pragma unroll
        for (int idx = g * kMfma / kReads; idx < (g + 1) * kMfma / kReads; ++idx) {
            const int i = idx / C::FN, j = idx % C::FN;
            acc[i][j] = MfmaF16F::op(cur.b[j], cur.a[i], acc[i][j]);   // D[n][t], as k_gemm
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <class C, int kVar, class AccArray>
__device__ __forceinline__ void outlier_gemm_pass(AccArray &accf, char *smem,
                                                  const EpilogueArgs &ep,
                                                  const int8_t *__restrict__ CB,
                                                  const int32_t *__restrict__ info,
                                                  const int32_t *__restrict__ groups,
                                                  const uint8_t *__restrict__ mask, int64_t m0,
                                                  int64_t n0, int64_t T, int64_t K, int64_t N,
                                                  int nout, int wm, int wn, int wave, int lane)
{
    using P = PassCfg<C>;
    static_assert(P::kLdsBytes <= C::kLdsBytes, "the pass's two stages fit the ring");
    constexpr int kBI = BStage<P, kVar>::kI;    // 16-byte code loads per lane per stage
    // (info, groups and mask are kernel arguments the kernel does not write,
    // so their uniform loads are scalar loads)
    const bool dense = info[2] == kOutDense;
    const int64_t ld = outlier_ld(nout);
    const int nst = dense ? info[1] : (int)(ld / 64);
    const char *abase = dense ? reinterpret_cast<const char *>(ep.X)
                              : reinterpret_cast<const char *>(ep.x_out);
    const int64_t lda = dense ? 2 * K : 2 * ld;
    const int8_t *bbase = dense ? CB : static_cast<const int8_t *>(ep.w_out);
    const int64_t ldb = dense ? K : ld;
    // first column (position) of stage st; stages past the last repeat it
    auto col = [&](int st) -> int {
        st = st < nst ? st : nst - 1;
        return dense ? 64 * groups[st] : 64 * st;
    };

    // A: direct loads into the stage's A region (the A half of Streams; its
    // B half is not used); B: codes through registers
    Streams<P> as;
    as.init(abase, lda, m0, T, abase, lda, m0, T, wave, lane);
    auto issue_a = [&](int buf, int st) {
        const int64_t kb = 2 * (int64_t)col(st);
        as.issue_a(smem, buf, kb, wave);
    };
    BStage<P, kVar> bs;
    bs.init(bbase, ldb, n0, N, ep, wave, lane);
    // stage st's B mask: 16 bits per lane, the outlier flags of its 16 columns
    auto mask16 = [&](int st) -> unsigned {
        if (!dense)
            return 0xffffu;
        const int q = groups[st < nst ? st : nst - 1];
        const unsigned long long m64 =
            *reinterpret_cast<const unsigned long long *>(mask + 8 * (int64_t)q);
        return (unsigned)(m64 >> (16 * (lane & 3))) & 0xffffu;
    };

    const int frow = (lane & 31) * P::ROWB;
    int fo[P::kKSteps];
#pragma unroll
    for (int ks = 0; ks < P::kKSteps; ++ks)
        fo[ks] = frow + (((2 * ks + (lane >> 5)) ^ P::swz(lane & 31)) << 4);
    const int aoff = wm * (P::BM / P::WM) * P::ROWB;
    const int boff = P::BM * P::ROWB + wn * (P::BN / P::WN) * P::ROWB;
    auto stage_a = [&](int buf) { return smem + buf * P::kStageBytes + aoff; };
    auto stage_b = [&](int buf) { return smem + buf * P::kStageBytes + boff; };

    auto none = [](auto, int) {};
    // Stage s: A in LDS buffer s % 2 by direct loads, B's codes in register
    // buffer s % 2.  Iteration kt issues B(kt+3) before its barrier and
    // A(kt+2) after it; both land by the next iteration's barrier, and the
    // codes of B(kt+1) are converted in iteration kt, during its MFMAs.
    // prologue: stage 0 complete in LDS buffer 0, B(1), B(2) and A(1) in flight
    bs.template load<0>(col(0));
    issue_a(0, 0);
    wait_vm<P::kAInstr>();                // B(0) landed
    auto masks = [&](unsigned m, unsigned (&bm)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bm[q] = byte_mask4((m >> (4 * q)) & 0xfu);
    };
    {
        const unsigned m = mask16(0);
        unsigned bm[4];
        masks(m, bm);
#pragma unroll
        for (int u = 0; u < BStage<P, kVar>::kUnits; ++u)
            bs.template store_unit<0>(smem, m, bm, u);
    }
    bs.template load<1>(col(1));
    bs.template load<0>(col(2));
    issue_a(1, 1);
    wait_vm<2 * kBI + P::kAInstr>();      // A(0) landed
    wait_lds();
    __builtin_amdgcn_s_barrier();
    Frags<P> f0, f1;
    read_frags<P>(f0, stage_a(0), stage_b(0), fo[0]);
    constexpr int kU = BStage<P, kVar>::kUnits;
    constexpr int kG = P::FM + P::FN;     // groups per k-step
    static_assert(kU <= 3 * kG, "conversion units fit three k-steps");
    // iteration kt with kt % 2 == B (compile time): stage kt in LDS buffer B,
    // B(kt+1) converted from register buffer 1-B into LDS buffer 1-B
    auto iter = [&](auto bc, int kt) {
        constexpr int B = decltype(bc)::value, NB = 1 - B;
        wait_vm<kBI + P::kAInstr>();      // B(kt+1) landed; B(kt+2), A(kt+1) may be in flight
        const unsigned m = mask16(kt + 1);
        unsigned bm[4];
        masks(m, bm);
        char *nstage = smem + NB * P::kStageBytes;   // its readers passed the last barrier
        // the conversion units spread evenly over the groups of three k-steps
        auto conv = [&](auto, int g, int base) {
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (u * 3 * kG / kU == base + g)
                    bs.template store_unit<NB>(nstage, m, bm, u);
        };
        pass_kstep<P>(f0, f1, stage_a(B), stage_b(B), fo[1], accf,
                      [&](auto z, int g) { conv(z, g, 0); });
        pass_kstep<P>(f1, f0, stage_a(B), stage_b(B), fo[2], accf,
                      [&](auto z, int g) { conv(z, g, kG); });
        pass_kstep<P>(f0, f1, stage_a(B), stage_b(B), fo[3], accf,
                      [&](auto z, int g) { conv(z, g, 2 * kG); });
        bs.template load<NB>(col(kt + 3));
        wait_vm<kBI>();                   // A(kt+1) landed; B(kt+3) may be in flight
        wait_lds();                       // stage kt read, B(kt+1) written
        __builtin_amdgcn_s_barrier();
        issue_a(B, kt + 2);
        pass_kstep<P>(f1, f0, stage_a(NB), stage_b(NB), fo[0], accf, none);
        // (the k-step above reads the first fragments of stage kt+1 from buffer
        // NB; on the last stage they are not used)
    };
    int kt = 0;
    for (; kt + 2 <= nst; kt += 2) {
        iter(std::integral_constant<int, 0>{}, kt);
        iter(std::integral_constant<int, 1>{}, kt + 1);
    }
    if (kt < nst)
        iter(std::integral_constant<int, 0>{}, kt);
    wait_vm<0>();   // the tail loads land before the buffers are reused
}

// More than 32 outlier columns: the int8 sums dequantized into fp32
// accumulators (the int32 ones die there, so the two share registers), the
// fp16 pass adding the outlier product onto them (outlier_gemm_pass), then
// the bias, one rounding, and the tile out through LDS like finish_tile's.
template <class C, bool kRelu, bool kZp, int kF8, class Acc = v16i>
__device__ __forceinline__ void outlier_pass(const Acc (&acc)[C::FM][C::FN],
                                             const float (&at)[C::FM], const int (&za)[C::FM],
                                             const int (&ra)[C::FM], char *smem,
                                             const EpilogueArgs &ep, const int8_t *CB,
                                             const int32_t *__restrict__ info,
                                             const int32_t *__restrict__ groups,
                                             const uint8_t *__restrict__ mask, int64_t m0,
                                             int64_t n0, int64_t T, int64_t K, int64_t N,
                                             int nout, int wm, int wn, int wave, int lane,
                                             int tid)
{
    const int tl = lane & 31, nl = 4 * (lane >> 5);
    const int64_t nw = n0 + wn * (C::BN / C::WN);
    v16f accf[C::FM][C::FN];
    if (nout < K) {
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            v4f sn[4];
            v4i zb[4], rb[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                int64_t n = nw + j * 32 + 8 * g + nl;
                n = n < N ? n : N - 4;
                sn[g] = *reinterpret_cast<const v4f *>(ep.scb + n);
                if constexpr (kZp) {
                    zb[g] = *reinterpret_cast<const v4i *>(ep.zp_b + n);
                    rb[g] = *reinterpret_cast<const v4i *>(ep.rs_b + n);
                }
            }
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if constexpr (kZp)
                        accf[i][j][r] = zp_dequant(acc[i][j][r], za[i], ra[i], zb[r / 4][r % 4],
                                                   rb[r / 4][r % 4], at[i], sn[r / 4][r % 4]);
                    else
                        accf[i][j][r] = (float)acc[i][j][r] * (at[i] * sn[r / 4][r % 4]);
                }
        }
    } else {   // every column an outlier: no int8 part
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    accf[i][j][r] = 0.0f;
    }
    __builtin_amdgcn_s_barrier();   // every wavefront is done reading the LDS ring
    outlier_gemm_pass<C, kF8 == kF8E4M3 ? kVarF8E4 : kF8 ? kVarF8 : kZp ? kVarZp : kVarAbsmax>(
        accf, smem, ep, CB, info, groups, mask, m0, n0, T, K, N, nout, wm, wn, wave, lane);
    static_assert(C::BM * C::BN * 2 <= C::kLdsBytes, "output tile fits the LDS ring");
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int tr = wm * (C::BM / C::WM) + i * 32 + tl;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                int64_t n = nw + j * 32 + 8 * g + nl;
                n = n < N ? n : N - 4;
                const uint2 bb = ep.bias ? *reinterpret_cast<const uint2 *>(ep.bias + n)
                                         : make_uint2(0u, 0u);
                const float bv[4] = {h2f((uint16_t)(bb.x & 0xffffu)), h2f((uint16_t)(bb.x >> 16)),
                                     h2f((uint16_t)(bb.y & 0xffffu)), h2f((uint16_t)(bb.y >> 16))};
                uint16_t h[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    h[q] = f2h_act<kRelu>(accf[i][j][4 * g + q] + bv[q]);
                const int u = (wn * (C::BN / C::WN) + j * 32 + 8 * g + nl) / 4;
                *reinterpret_cast<uint2 *>(smem + tr * (C::BN * 2) + 8 * (u ^ (tr & 31))) =
                    make_uint2((unsigned)h[0] | ((unsigned)h[1] << 16),
                               (unsigned)h[2] | ((unsigned)h[3] << 16));
            }
        }
    }
    __syncthreads();
    write_tile<C>(smem, ep, m0, n0, T, N, tid);
}

// One tile of the int8 GEMM with the up-to-32-outlier epilogue (or the raw
// int32 store); smem: the ring, then (output path) the tile's outlier rows.
// kBiasSel: -1 picks the epilogue with or without the bias per call (ep.bias);
// 0 / 1 compile only the one without / with it.  A kernel with both epilogues
// has the compiler hoist the accumulators' int-to-float conversions, which
// both begin with, above the branch, where they outlive the registers free
// there and spill (measured on the 2 x 4 wavefront shape: 52 bytes per lane,
// reloaded inside the epilogue behind full memory waits).
template <class C, bool kRawI32, bool kRelu, bool kZp, int kF8, int kBiasSel = -1>
__device__ __forceinline__ void gemm_tile(char *smem, const int8_t *__restrict__ A,
                                          const int8_t *__restrict__ B, int64_t T, int64_t K,
                                          int64_t N, const EpilogueArgs &ep)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int ntm = (int)((T + C::BM - 1) / C::BM), ntn = (int)((N + C::BN - 1) / C::BN);
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, ntm, ntn, C::GROUP, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;

    // More than 32 outlier columns: k_gemm_many computes this output.
    const int nout = kRawI32 ? 0 : *ep.n_out;
    if (!kRawI32 && nout > kOutlierPad)
        return;
    // the outlier rows do not depend on the GEMM: staged into LDS now, they
    // have landed when the main loop starts (its first wait covers them)
    char *orows = smem + C::kLdsBytes;
    if constexpr (!kRawI32)
        issue_outlier_rows<C>(orows, ep, m0, n0, T, N, wave, lane);

    using Acc = std::conditional_t<kF8 != kF8None, v16f, v16i>;
    Acc acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0;

    {
        Streams<C> st;
        st.init(reinterpret_cast<const char *>(A), K, m0, T, reinterpret_cast<const char *>(B), K,
                n0, N, wave, lane);
        if constexpr (kF8 != kF8None)
            mainloop_f8<C, kF8>(smem, st, (int)(K / C::ROWB), acc, wm, wn, wave, lane);
        else
            run_mainloop<C, MfmaI8>(smem, st, (int)(K / C::ROWB), acc, wm, wn, wave, lane);
    }

    // The MFMAs compute D = CB_tile * Xq_tile^T, so a 32x32 accumulator holds
    // C transposed: lane l has output row t = lane%32 of the sub-tile and, in
    // registers 4g..4g+3, the four consecutive output columns
    // n = 8g + 4*(lane/32) + {0,1,2,3}.  Each lane therefore needs one row
    // scale per sub-tile row and writes 4 adjacent outputs with one store.
    const int tl = lane & 31, nl = 4 * (lane >> 5);
    const int64_t tw = m0 + wm * (C::BM / C::WM), nw = n0 + wn * (C::BN / C::WN);
    if constexpr (kRawI32) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int64_t t = tw + i * 32 + tl;
            if (t >= T)
                continue;
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t n = nw + j * 32 + 8 * g + nl;
                    if (n < N)
                        *reinterpret_cast<v4i *>(ep.c_i32 + t * N + n) =
                            v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                acc[i][j][4 * g + 3]};
                }
        }
    } else {
        float at[C::FM];
        int za[C::FM], ra[C::FM];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int64_t t = tw + i * 32 + tl;
            if constexpr (kZp)
                zp_row(ep, t < T ? t : T - 1, K, at[i], za[i], ra[i]);
            else if constexpr (kF8 != kF8None)
                at[i] = ep.a[t < T ? t : T - 1];   // the row scale 2^-e
            else
                at[i] = ep.a[t < T ? t : T - 1] * (1.0f / 16129.0f);
        }
        if (kBiasSel == 1 || (kBiasSel < 0 && ep.bias))
            finish_tile<C, kBiasSel != 0, kRelu, kZp, Acc>(acc, at, za, ra, orows, smem, ep, m0,
                                                           n0, T, N, nout, wm, wn, lane, tid);
        else
            finish_tile<C, false, kRelu, kZp, Acc>(acc, at, za, ra, orows, smem, ep, m0, n0, T, N,
                                                   nout, wm, wn, lane, tid);
    }
}

// More than 32 outlier columns (k_gemm returns at once then, and this path
// runs otherwise): per tile the int8 GEMM (skipped when every column is an
// outlier, e.g. threshold 0, since Xq is then all zeros), then the fused
// fp16 pass over the outlier columns.  A kernel of its own (k_gemm_many)
// where k_gemm runs another tile shape, so that the registers this path
// needs do not cost k_gemm's epilogue; one launch with k_gemm (k_gemm_both)
// where both run the same shape; one tile per block (a persistent tile loop
// makes the compiler spill around it).  smem is the ring.
template <class C, bool kRelu, bool kZp, int kF8>
__device__ __forceinline__ void many_tile(char *smem, const int8_t *__restrict__ A,
                                          const int8_t *__restrict__ B, int64_t T, int64_t K,
                                          int64_t N, const EpilogueArgs &ep,
                                          const int32_t *__restrict__ info,
                                          const int32_t *__restrict__ groups,
                                          const uint8_t *__restrict__ mask, int nout)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int ntm = (int)((T + C::BM - 1) / C::BM), ntn = (int)((N + C::BN - 1) / C::BN);
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, ntm, ntn, C::GROUP, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;

    using Acc = std::conditional_t<kF8 != kF8None, v16f, v16i>;
    Acc acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0;
    if (nout < K) {
        // kept-column mode (absmax and FP8; info[3] = kc > 0): the 8-bit
        // product over the kc compacted kept columns, at the start of each Xq
        // row and in ep.cb_kept [N, kc]; the outlier columns' products are all
        // 0 (int8 code 0, FP8 code +0)
        int64_t kk = K;
        const int8_t *Bk = B;
        if constexpr (!kZp) {
            const int kc = info[3];
            if (kc > 0) {
                kk = kc;
                Bk = ep.cb_kept;
            }
        }
        Streams<C> st;
        st.init(reinterpret_cast<const char *>(A), K, m0, T, reinterpret_cast<const char *>(Bk),
                kk, n0, N, wave, lane);
        if constexpr (kF8 != kF8None)
            mainloop_f8<C, kF8>(smem, st, (int)(kk / C::ROWB), acc, wm, wn, wave, lane);
        else
            run_mainloop<C, MfmaI8>(smem, st, (int)(kk / C::ROWB), acc, wm, wn, wave, lane);
    }
    float at[C::FM];
    int za[C::FM], ra[C::FM];
    const int64_t tw = m0 + wm * (C::BM / C::WM) + (lane & 31);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t t = tw + i * 32;
        if constexpr (kZp)
            zp_row(ep, t < T ? t : T - 1, K, at[i], za[i], ra[i]);
        else if constexpr (kF8 != kF8None)
            at[i] = ep.a[t < T ? t : T - 1];
        else
            at[i] = ep.a[t < T ? t : T - 1] * (1.0f / 16129.0f);
    }
    outlier_pass<C, kRelu, kZp, kF8, Acc>(acc, at, za, ra, smem, ep, B, info, groups, mask, m0, n0,
                                          T, K, N, nout, wm, wn, wave, lane, tid);
}

template <class C, bool kRawI32, bool kRelu, bool kZp = false, int kF8 = kF8None>
__global__ __launch_bounds__(C::kThreads) void k_gemm(const int8_t *__restrict__ A,
                                                      const int8_t *__restrict__ B, int64_t T,
                                                      int64_t K, int64_t N, EpilogueArgs ep)
{
    __shared__ __attribute__((aligned(1024)))
    char smem[C::kLdsBytes + (kRawI32 ? 0 : OutlierRows<C>::kBytes)];
    gemm_tile<C, kRawI32, kRelu, kZp, kF8>(smem, A, B, T, K, N, ep);
}

template <class C, bool kRelu, bool kZp = false, int kF8 = kF8None>
__global__ __launch_bounds__(C::kThreads) void k_gemm_many(
    const int8_t *__restrict__ A, const int8_t *__restrict__ B, int64_t T, int64_t K, int64_t N,
    EpilogueArgs ep, const int32_t *__restrict__ info, const int32_t *__restrict__ groups,
    const uint8_t *__restrict__ mask)
{
    const int nout = info[0];
    if (nout <= kOutlierPad)
        return;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
    many_tile<C, kRelu, kZp, kF8>(smem, A, B, T, K, N, ep, info, groups, mask, nout);
}

// Both output paths in one launch, the path chosen per call from the outlier
// count on the device: when both run in the same tile shape (and so the same
// register budget), this saves the second, idle launch.  One kernel per bias
// choice (see gemm_tile's kBiasSel).
template <class C, bool kRelu, bool kBias>
__global__ __launch_bounds__(C::kThreads) void k_gemm_both(
    const int8_t *__restrict__ A, const int8_t *__restrict__ B, int64_t T, int64_t K, int64_t N,
    EpilogueArgs ep, const int32_t *__restrict__ info, const int32_t *__restrict__ groups,
    const uint8_t *__restrict__ mask)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes + OutlierRows<C>::kBytes];
    const int nout = info[0];
    if (nout > kOutlierPad)
        many_tile<C, kRelu, false, false>(smem, A, B, T, K, N, ep, info, groups, mask, nout);
    else
        gemm_tile<C, false, kRelu, false, false, kBias ? 1 : 0>(smem, A, B, T, K, N, ep);
}

// The int8 GEMM (K must be a multiple of C::ROWB) with its fused epilogue
// (and the output activation, ep.act, a template parameter of the output
// kernels); for the output (not the raw int32 sums) also k_gemm_many, of
// which only one does work, depending on the outlier count on the device.
template <class C, class CM = C>
hipError_t launch(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                  const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0 = nullptr,
                  hipEvent_t ev1 = nullptr)
{
    static_assert(C::BM == CM::BM && C::BN == CM::BN && C::ROWB == CM::ROWB, "one tile grid");
    if (K % C::ROWB != 0)
        return hipErrorInvalidValue;
    const int64_t ntm = (T + C::BM - 1) / C::BM, ntn = (N + C::BN - 1) / C::BN;
    const dim3 grid((unsigned)(ntm * ntn));
    if (ev0) {
        const hipError_t e = hipEventRecord(ev0, s);
        if (e != hipSuccess)
            return e;
    }
    // absmax output with both paths in the same 128-byte-stage shape: one
    // launch (measured: 261 -> 259 us at 4096 x 4096 x 16384, 53.4 -> 52.0 us at
    // 2048 x 2048 x 8192; the 64-byte-stage shape spills more combined)
    if constexpr (std::is_same_v<C, CM> && C::ROWB == 128) {
        if (!ep.c_i32 && !ep.f8 && !ep.row_zp) {
            if (ep.act && ep.bias)
                hipLaunchKernelGGL((k_gemm_both<C, true, true>), grid, dim3(C::kThreads), 0, s, Xq,
                                   CB, T, K, N, ep, ep.n_out, ep.groups, ep.mask);
            else if (ep.act)
                hipLaunchKernelGGL((k_gemm_both<C, true, false>), grid, dim3(C::kThreads), 0, s,
                                   Xq, CB, T, K, N, ep, ep.n_out, ep.groups, ep.mask);
            else if (ep.bias)
                hipLaunchKernelGGL((k_gemm_both<C, false, true>), grid, dim3(C::kThreads), 0, s,
                                   Xq, CB, T, K, N, ep, ep.n_out, ep.groups, ep.mask);
            else
                hipLaunchKernelGGL((k_gemm_both<C, false, false>), grid, dim3(C::kThreads), 0, s,
                                   Xq, CB, T, K, N, ep, ep.n_out, ep.groups, ep.mask);
            if (ev1) {
                const hipError_t e = hipEventRecord(ev1, s);
                if (e != hipSuccess)
                    return e;
            }
            return hipGetLastError();
        }
    }
    if (ep.c_i32)
        hipLaunchKernelGGL((k_gemm<C, true, false>), grid, dim3(C::kThreads), 0, s, Xq, CB, T, K,
                           N, ep);
    else if (ep.f8 == kF8E4M3)
        hipLaunchKernelGGL((k_gemm<C, false, false, false, kF8E4M3>), grid, dim3(C::kThreads), 0,
                           s, Xq, CB, T, K, N, ep);
    else if (ep.f8)
        hipLaunchKernelGGL((k_gemm<C, false, false, false, kF8E5M2>), grid, dim3(C::kThreads), 0,
                           s, Xq, CB, T, K, N, ep);
    else if (ep.row_zp)
        hipLaunchKernelGGL((k_gemm<C, false, false, true>), grid, dim3(C::kThreads), 0, s, Xq, CB,
                           T, K, N, ep);
    else if (ep.act)
        hipLaunchKernelGGL((k_gemm<C, false, true>), grid, dim3(C::kThreads), 0, s, Xq, CB, T, K,
                           N, ep);
    else
        hipLaunchKernelGGL((k_gemm<C, false, false>), grid, dim3(C::kThreads), 0, s, Xq, CB, T, K,
                           N, ep);
    if (ev1) {
        const hipError_t e = hipEventRecord(ev1, s);
        if (e != hipSuccess)
            return e;
    }
    if (!ep.c_i32) {
        if (ep.f8 == kF8E4M3)
            hipLaunchKernelGGL((k_gemm_many<CM, false, false, kF8E4M3>), grid, dim3(CM::kThreads),
                               0, s, Xq, CB, T, K, N, ep, ep.n_out, ep.groups, ep.mask);
        else if (ep.f8)
            hipLaunchKernelGGL((k_gemm_many<CM, false, false, kF8E5M2>), grid, dim3(CM::kThreads),
                               0, s, Xq, CB, T, K, N, ep, ep.n_out, ep.groups, ep.mask);
        else if (ep.row_zp)
            hipLaunchKernelGGL((k_gemm_many<CM, false, true>), grid, dim3(CM::kThreads), 0, s, Xq, CB,
                               T, K, N, ep, ep.n_out, ep.groups, ep.mask);
        else if (ep.act)
            hipLaunchKernelGGL((k_gemm_many<CM, true>), grid, dim3(CM::kThreads), 0, s, Xq, CB, T, K,
                               N, ep, ep.n_out, ep.groups, ep.mask);
        else
            hipLaunchKernelGGL((k_gemm_many<CM, false>), grid, dim3(CM::kThreads), 0, s, Xq, CB, T,
                               K, N, ep, ep.n_out, ep.groups, ep.mask);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace gemm
}  // namespace llmint8
