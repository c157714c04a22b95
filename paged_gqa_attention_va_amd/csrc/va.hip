// va.hip -- paged GQA target-verify attention for MI355X (gfx950 / CDNA4).
//
// The kernels and the host side of the C ABI declared in include/va.h.
//
//  va_split_kv_fp8_w4_kernel   Split-KV main kernel for an FP8 e4m3 cache,
//      paged layout, when a workgroup streams enough pages: one wave per SIMD,
//      each wave a key group holding every packed row (Q operands in registers,
//      O^T in accumulation registers), its own LDS ring and no barrier inside
//      the page loop; the four key groups are combined in the epilogue.
//  va_split_kv_fp8_w8_kernel   The FP8 main kernel with two waves per SIMD (4
//      key groups x 2 row groups, a shared ring stage per key group): shorter
//      prologue and epilogue, for workgroups with few pages, and the prefix +
//      extend layout.
//  va_split_kv_bf16_w8_kernel  The same for a bf16 cache.
//      Each workgroup takes a contiguous share of the flattened page space of
//      all (sequence, kv head) pairs.  For each piece it copies every K/V page
//      once, straight from HBM into an LDS ring, and reuses it for all G*q_len
//      packed query rows (GQA packing); MFMA QK^T and PV with an online
//      softmax; then either the final rows or a partial (o, lse) per piece.
//      A template flag of the w8 kernels selects the paged layout (block table)
//      or the prefix + extend layout (keys gathered row by row through
//      kv_indices, draft keys from separate buffers).
//  va_mla_split_kernel  The same split for absorbed MLA: 576-wide cache rows
//                       (latent + RoPE part), values = the 512-wide latent.
//  va_merge_kernel      Segment reduce: log-sum-exp merge of the partials of
//                       every (sequence, kv head) that was split over
//                       workgroups (256- or 512-wide rows).
//  va_spec_block_table_kernel, va_validate_kernel, va_fp8_to_bf16_kernel
//                       draft-extend metadata, validate mode, test helper.
//  va_stream_pages_kernel  Diagnostic: the FP8 kernels' copy path alone (the
//                       streaming ceiling).
//
// The method comes from the sglang PR #36330 summary page ("Implementation
// breakdown", item 1: pack the G query heads and speculative tokens of a group
// so each loaded KV tile serves all of them, split the KV range into segments
// for CU parallelism, merge in a reduce-segments kernel).  The sglang PR #34517
// summary page says the same in "Motivation": one KV-tile load per group of
// query heads.  The kernels here are a CDNA4 design of their own, not the
// Triton ones.
//
// Layout of the packed rows of one (sequence b, kv head g): row r = t*G + h
// (t = speculative token, h = head within the group), padded to 16-row MFMA
// tiles.  Each wave computes S^T = K Q^T and O^T = V^T P^T, so
//   - the S^T accumulator already is the P^T B-operand, so no shuffle is needed;
//   - row statistics (max, sum) stay inside one lane column.
//
// Stream-K partition: WG w of N handles the pages between cost positions
// floor(w*T/N) and floor((w+1)*T/N), where T is the pages of all pairs plus a
// fixed cost for each pair that starts inside a share (see locate), computed on
// the device from seqused_k / cu_seqlens_q.  Any length mix therefore balances
// over the CUs with no host-side lengths (graph-safe).  Only a WG's first and
// last piece can be split: they write their partials to workspace slots 2w and
// 2w + 1.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "va.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx8_t __attribute__((ext_vector_type(8)));

constexpr int kHeadDim = 256;
constexpr int kPage = 16;
constexpr int kThreads = 256;            // merge and helper kernels: 4 waves of 64
// Online-softmax rescale threshold (log2 units).  The running max m is only
// moved when a new logit exceeds it by more than kTau.  Then p = 2^(x - m) <= 2^8
// and O, l stay exact up to rounding; the final O/l does not depend on m.
constexpr float kTau = 8.0f;
constexpr int kKvFp8 = 0;
constexpr int kKvBf16 = 1;

struct SplitParams {
    const uint16_t *q;
    const uint8_t *k;
    const uint8_t *v;
    const int32_t *bt;
    const int32_t *cu;
    const int32_t *seqused;
    const float *kdesc;
    const float *vdesc;
    uint16_t *out;
    void *ws_o;           // [2 grid][rows_max][256]: fp16 (FP8 cache) or fp32 (bf16 cache);
                          // slot 2 w = workgroup w's first piece, 2 w + 1 its last (only
                          // those two pieces of a workgroup can be split)
    float *ws_lse;        // [2 grid][rows_max]   log2-domain LSE of the scaled logits
    int32_t *ws_prefix;   // [BH + 1] exclusive prefix of page counts, [BH] = total
    int32_t *ws_cost;     // [BH + 1] exclusive prefix of the pairs' costs (see locate)
    int32_t *ws_meta;     // [0] = workgroups in use
    int32_t piece_cost;   // pages charged for a pair that starts inside a workgroup's range
    float scale_log2;     // softmax_scale * log2(e)
    float cap_log2;       // logit softcap * log2(e) (0 = no softcap)
    const float *sinks;   // [Hq] sink logits (natural-log units) or null
    int32_t window_left;  // sliding window: keys from i - window_left on (-1 = none)
    int32_t num_seqs, hq, hkv, log2g, mbps, grid_n, min_pages, rows_max;
    int32_t total_q, max_q;   // rows of q / out, and the longest valid query block
    int64_t num_blocks;
    // prefix + extend layout (kv_indptr == null: paged layout).  Key j < P of
    // sequence b is row kv_indices[kv_indptr[b] + j] of the k / v buffers
    // ([num_rows, Hkv, 256]); key P + i is row cu[b] + i of kext / vext.
    const int32_t *kv_indptr;
    const int32_t *kv_indices;
    const uint8_t *kext;
    const uint8_t *vext;
    int64_t num_indices;  // elements of kv_indices
    int64_t num_rows;     // rows of the k / v buffers
    unsigned long long *stamps;   // phase timestamps (library built with VA_STAMPS), else null
};

struct MergeParams {
    const int32_t *cu;
    const float *vdesc;
    const float *sinks;   // [Hq] sink logits (natural-log units) or null
    const void *ws_o;     // fp16 or fp32 partials, see SplitParams
    const float *ws_lse;
    const int32_t *ws_prefix;
    const int32_t *ws_cost;
    const int32_t *ws_meta;
    uint16_t *out;
    int32_t num_seqs, hq, hkv, log2g, max_q, rows_max, total_q;
};

// ------------------------------------------------------ phase timestamps --
//
// A library built with -DVA_STAMPS records, per wave of the one-wave-per-SIMD
// FP8 kernel, the constant 100 MHz clock (s_memrealtime) at phase boundaries
// into the buffer given to va_set_stamp_buffer: kStampSlots 64-bit words per
// wave, wave (w, kg) at ((w * 4 + kg) * kStampSlots).  Slots: 0 entry,
// 1 work located, 2 own Q rows landed, 3 Q operands in registers, 4 first
// step's pages landed, 5 second step's pages landed, 6 page loop done, 7
// epilogue done (these six for the workgroup's first piece), 8 exit, 9 steps
// of the first piece, 10 pieces, 11 XCD of the workgroup, 12 page-loop passes
// of the first piece, 13..15 the epilogue of the first piece: row states
// exchanged, scaled O published, all published; 16..19 the middle step
// (nst / 2) of the first piece's first pass: its K landed, QK and softmax
// done, its V landed, PV done; 20, 21 the shader clock counter (s_memtime) at
// that step's K landing and PV end.  Stamps taken inside the page loop (4, 5,
// 16..21) keep the low 32 bits only, held in registers and written after the
// loop: a store there would be counted by the vmcnt waits of the copy ring.
// Without VA_STAMPS the statements compile to nothing.
constexpr int kStampSlots = 32;
#ifdef VA_STAMPS
#define VA_STAMP(p, w, kg, lane, k, value)                                                   \
    do {                                                                                 \
        if ((p).stamps && (lane) == 0)                                                   \
            (p).stamps[((int64_t)(w) * 4 + (kg)) * kStampSlots + (k)] = (value);        \
    } while (0)
#define VA_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define VA_STAMP(p, w, kg, lane, k, value) \
    do {                                   \
    } while (0)
#define VA_NOW() 0ull
#endif

// ------------------------------------------------------------ primitives --

__device__ __forceinline__ uint32_t fp8x2_lo_to_bf16x2(uint32_t w)
{
    // bytes 0,1 of w (two e4m3fn values) -> two bf16 (exact: every e4m3fn
    // value is a bf16 value).  Scale 1.0 = no scaling.
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

__device__ __forceinline__ uint32_t fp8x2_hi_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// v_perm_b32: byte i of the result = byte sel.i of the 8-byte value {hi, lo}
// (selector 0..3 = bytes of lo, 4..7 = bytes of hi).
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf16x2_t v;
    v[0] = (__bf16)a;    // round to nearest even (v_cvt_pk_bf16_f32)
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ floatx4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const floatx4_t &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 MFMA with fp8 e4m3 A and B (format code 0 for both), unit
// block scales (E8M0 127 = 2^0).  Lane l holds 32 k-values of row/column l%16.
__device__ __forceinline__ floatx4_t mfma16_f8(const intx8_t &a, const intx8_t &b, const floatx4_t &c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Inclusive prefix sum over the wave with DPP moves: row_shr 1, 2, 4, 8 scan
// each row of 16 lanes, then row_bcast 15 and 31 add the totals of the rows
// before (lanes a move does not reach take the 0 of `old`).
__device__ __forceinline__ int wave_scan_dpp(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return x;
}

__device__ __forceinline__ float exp2_fast(float x)
{
    return __builtin_amdgcn_exp2f(x);      // v_exp_f32; exp2(-inf) = 0
}

// Maxima of values that come out of inline assembly: written as instructions
// so that no canonicalising v_max x, x is put in front of each operand (the
// inputs are never NaN where these are used).
// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one row of a
// 16-row MFMA tile).  A swizzle swaps the 16-lane halves of each 32-lane half
// (no address register); the 32-lane step permutes with an address formed on
// the spot from an opaque lane index, so that it is not formed once and held
// (or spilled) for the whole kernel.  Bit for bit the two xor shuffles.
__device__ __forceinline__ float xor16_lane(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

__device__ __forceinline__ float xor32_lane(float x)
{
    int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float row4_max(float x)
{
    x = fmaxf(x, xor16_lane(x));
    return fmaxf(x, xor32_lane(x));
}

__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float max2f(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ int uniform(int x)
{
    return __builtin_amdgcn_readfirstlane(x);
}

// Load of a read-only int32 at a wave-uniform address through the constant
// address space, so it becomes a scalar load (it then waits on lgkmcnt, never
// on the vmcnt that tracks the LDS ring's copies).
__device__ __forceinline__ int load_uniform(const int32_t *base, int64_t idx)
{
    typedef const __attribute__((address_space(4))) int32_t cint32;
    return ((cint32 *)base)[idx];
}

// Three scalar loads under one wait: a[0..2] are uniform addresses.  Written
// out because the compiler, short of scalar registers, may otherwise give each
// load a wait of its own, a memory latency apiece.
__device__ __forceinline__ void load_uniform3(int (&v)[3], const int32_t *a0, const int32_t *a1, const int32_t *a2)
{
    asm volatile("s_load_dword %0, %3, 0x0\n\t"
                 "s_load_dword %1, %4, 0x0\n\t"
                 "s_load_dword %2, %5, 0x0\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&s"(v[0]), "=&s"(v[1]), "=&s"(v[2])
                 : "s"(a0), "s"(a1), "s"(a2)
                 : "memory");
}

// Ten block-table entries row[min(first + i, last)], i = 0..9, under one wait
// (the same reason as load_uniform3).  first <= last, both within the row.
__device__ __forceinline__ void load_entries10(int (&v)[10], const int32_t *row, int first, int last)
{
    const int32_t *a[10];
#pragma unroll
    for (int i = 0; i < 10; ++i)
        a[i] = row + min(first + i, last);
    asm volatile("s_load_dword %0, %10, 0x0\n\t"
                 "s_load_dword %1, %11, 0x0\n\t"
                 "s_load_dword %2, %12, 0x0\n\t"
                 "s_load_dword %3, %13, 0x0\n\t"
                 "s_load_dword %4, %14, 0x0\n\t"
                 "s_load_dword %5, %15, 0x0\n\t"
                 "s_load_dword %6, %16, 0x0\n\t"
                 "s_load_dword %7, %17, 0x0\n\t"
                 "s_load_dword %8, %18, 0x0\n\t"
                 "s_load_dword %9, %19, 0x0\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&s"(v[0]), "=&s"(v[1]), "=&s"(v[2]), "=&s"(v[3]), "=&s"(v[4]),
                   "=&s"(v[5]), "=&s"(v[6]), "=&s"(v[7]), "=&s"(v[8]), "=&s"(v[9])
                 : "s"(a[0]), "s"(a[1]), "s"(a[2]), "s"(a[3]), "s"(a[4]),
                   "s"(a[5]), "s"(a[6]), "s"(a[7]), "s"(a[8]), "s"(a[9])
                 : "memory");
}

// A descale factor (one float, or 1 when the pointer is null) through the
// scalar cache: the value then lives in a scalar register.  A vector-register
// copy can be spilled, and its reload waits for every copy in flight.
__device__ __forceinline__ float load_descale(const float *ptr)
{
    return ptr ? __builtin_bit_cast(float, load_uniform(reinterpret_cast<const int32_t *>(ptr), 0)) : 1.0f;
}

// Pages of (sequence, kv head) bg that hold keys for at least one query row.
// Clamped to the block-table row so a bad length cannot index past it.
// First page any query row of a sequence can see: with a sliding window the
// lowest visible key is that of query token 0, (lk - lq) - window_left.
__device__ __forceinline__ int first_page(int lk, int lq, int wl)
{
    return wl < 0 ? 0 : max(0, lk - lq - wl) / kPage;
}

// Query length of a sequence whose rows are [q0, q1).  A range that leaves
// [0, total_q) or is longer than max_q counts as empty, so no cu_seqlens_q
// value can move a q read or an out write outside those buffers.
__device__ __forceinline__ int checked_q_len(int q0, int q1, int total_q, int max_q)
{
    return (q0 >= 0 && q1 >= q0 && q1 <= total_q && q1 - q0 <= max_q) ? q1 - q0 : 0;
}

// Keys of a sequence from its prefix range [s0, s1) of kv_indices and its
// (checked) query length, in the prefix + extend layout.  A prefix range
// outside kv_indices counts as an empty sequence.
__device__ __forceinline__ int prefix_keys(int s0, int s1, int lq, int64_t num_indices)
{
    return (s0 >= 0 && s1 >= s0 && s1 <= num_indices) ? (s1 - s0) + lq : 0;
}

// Pages of (sequence, kv head) bg that the split covers: first_page .. the
// last page holding a key below the sequence's key count (clamped to the
// block-table row).  In the prefix + extend layout a "page" is 16 consecutive
// keys of the sequence.
// The loaded words are also returned: cu_seqlens_q[b], cu_seqlens_q[b + 1] and
// seqused_k[b] (paged layout; the key count in the prefix + extend layout).
__device__ __forceinline__ int pages_of(const SplitParams &p, int bg, int &q0, int &q1, int &lk)
{
    const int b = bg / p.hkv;
    q0 = p.cu[b];
    q1 = p.cu[b + 1];
    const int lq = checked_q_len(q0, q1, p.total_q, p.max_q);
    lk = p.kv_indptr ? prefix_keys(p.kv_indptr[b], p.kv_indptr[b + 1], lq, p.num_indices) : p.seqused[b];
    if (lq <= 0 || lk <= 0)
        return 0;
    return max(0, min((lk + kPage - 1) / kPage, p.mbps) - first_page(lk, lq, p.window_left));
}

__device__ __forceinline__ int pages_of(const SplitParams &p, int bg)
{
    int q0, q1, lk;
    return pages_of(p, bg, q0, q1, lk);
}

__device__ __forceinline__ uint32_t u4get(const uint4 &u, int i)
{
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// ------------------------------------------------------- per-step compute --

// Per-wave softmax state of its row tiles.
template <int RTW>
struct RowState {
    floatx4_t o[16][RTW];   // O^T tiles: o[t][rt][e] = O[row l%16][dim 16*(4*(l/16)+e) + t]
    float m[RTW];           // running max, log2-scaled logits
    float l[RTW];           // this lane's partial sum of 2^(x - m)
};


// Softmax part of a 32-key step: online softmax on S^T; returns the P^T
// B-operands (bf16) of this wave's row tiles.
//   masked  this step holds keys some row may not see (the causal tail, keys
//           at or past seqused_k, or a missing second page); uniform
//   limit   per row tile: the last key index row (lane%16) may see; with a
//           sliding window the first is limit - window_left (wlim)
//   key0    index of key 0 of page a; has_b: page b is part of this piece
//   c       per row tile: logit multiplier (softmax_scale * k_descale * log2 e,
//           times the row's Q scale where Q was rescaled)
// Logit softcap in log2 units: x = C tanh(x / C) with C = softcap log2(e),
// tanh(y) = 1 - 2 / (e^(2y) + 1) (saturates to +-C; -inf stays -inf).
__device__ __forceinline__ float softcap_log2(float x, float C)
{
    const float e = exp2_fast(x * (2.8853900817779268f / C));     // e^(2 x / C) = 2^(2 log2(e) x / C)
    return C - (2.0f * C) * __builtin_amdgcn_rcpf(e + 1.0f);      // v_rcp_f32 (1 ulp): rcp(inf) = 0
}

template <int RTW, bool CAP>
__device__ __forceinline__ void softmax_step(RowState<RTW> &st, bf16x8_t (&pop)[RTW],
                                             const floatx4_t (&S)[2][RTW], const int (&limit)[RTW],
                                             uint32_t wlim, int key0, bool has_b, const float (&c)[RTW],
                                             float cap, int lane, bool masked)
{
    const int j = lane >> 4;
    // Logits in log2 units, masked by select (NaN garbage in masked slots is
    // dropped).  The running max m of a row only moves when a logit exceeds it
    // by more than kTau, so in the common case each lane only compares its own
    // logits with m + kTau and one wave-wide vote decides; the cross-lane row
    // max and the rescale of O and l run only when the vote says so.
    float x[RTW][8];
    bool need_any = false;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = S[a][rt][e] * c[rt];
                if constexpr (CAP)
                    v = softcap_log2(v, cap);
                if (masked) {
                    // visible: limit - window_left <= key <= limit (wlim = window_left, or 2^31 - 1)
                    const int key = key0 + 16 * a + 4 * j + e;
                    const bool ok = (a == 0 || has_b) && (uint32_t)(limit[rt] - key) <= wlim;
                    v = ok ? v : -INFINITY;
                }
                x[rt][4 * a + e] = v;
            }
        const float lmax = fmaxf(fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3])),
                                 fmaxf(fmaxf(x[rt][4], x[rt][5]), fmaxf(x[rt][6], x[rt][7])));
        need_any |= lmax > st.m[rt] + kTau;
    }
    if (__any(need_any)) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            float t = x[rt][0];
#pragma unroll
            for (int i = 1; i < 8; ++i)
                t = fmaxf(t, x[rt][i]);
            t = fmaxf(t, __shfl_xor(t, 16));
            t = fmaxf(t, __shfl_xor(t, 32));            // row max of this step
            const bool need = t > st.m[rt] + kTau;
            const float alpha = need ? exp2_fast(st.m[rt] - t) : 1.0f;
            st.m[rt] = need ? t : st.m[rt];
            st.l[rt] *= alpha;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt)
                st.o[tt][rt] *= alpha;
        }
    }

#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const float mref = st.m[rt] == -INFINITY ? 0.0f : st.m[rt];
        float p[8];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = exp2_fast(x[rt][i] - mref);
            sum += p[i];
        }
        st.l[rt] += sum;
        uint4 w;
        w.x = pack_bf16x2(p[0], p[1]);
        w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]);
        w.w = pack_bf16x2(p[6], p[7]);
        pop[rt] = __builtin_bit_cast(bf16x8_t, w);
    }
}

// Keys of a step whose V rows must be zeroed before PV: at or past seqused_k
// (they may hold NaN bytes), or in page b when page b is not part of the
// piece.  Bit e = key (page e/4, slot 4j + e%4) of this lane.
__device__ __forceinline__ uint32_t v_zero_mask(int key0, bool has_b, int key_end, int lane)
{
    const int j = lane >> 4;
    uint32_t z = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int key = key0 + 16 * (e >> 2) + 4 * j + (e & 3);
        if (key >= key_end || (e >= 4 && !has_b))
            z |= 1u << e;
    }
    return z;
}


// PV with FP8 V rows read from a ring stage, 8 bytes (dims 8h .. 8h+7 of the
// lane's 16) of each of the 8 keys at a time, so only 16 registers of raw V
// are live.  Same operand order as pv_regs.
template <int RTW>
__device__ __forceinline__ void pv_lds(RowState<RTW> &st, const unsigned char *stage,
                                       const bf16x8_t (&pop)[RTW], bool masked, uint32_t zmask, int lane)
{
    const int m = lane & 15, j = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint2 vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int n = 4 * j + (e & 3);
            vv[e] = *reinterpret_cast<const uint2 *>(stage + 8192 + 4096 * (e >> 2) + 256 * n +
                                                     16 * (m ^ n) + 8 * h);
        }
        if (masked) {                                  // wave-uniform
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (zmask & (1u << e))
                    vv[e] = make_uint2(0, 0);
        }
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * h + qq;
            uint32_t A[4][4];
#pragma unroll
            for (int kp = 0; kp < 4; ++kp) {
                const uint32_t X = qq ? vv[2 * kp].y : vv[2 * kp].x;
                const uint32_t Y = qq ? vv[2 * kp + 1].y : vv[2 * kp + 1].x;
                const uint32_t lo = byte_perm(Y, X, 0x05010400u);   // X0 Y0 X1 Y1
                const uint32_t hi = byte_perm(Y, X, 0x07030602u);   // X2 Y2 X3 Y3
                A[0][kp] = fp8x2_lo_to_bf16x2(lo);
                A[1][kp] = fp8x2_hi_to_bf16x2(lo);
                A[2][kp] = fp8x2_lo_to_bf16x2(hi);
                A[3][kp] = fp8x2_hi_to_bf16x2(hi);
            }
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) {
                const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(A[xx][0], A[xx][1], A[xx][2], A[xx][3]));
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
                    st.o[4 * q + xx][rt] = mfma16(vop, pop[rt], st.o[4 * q + xx][rt]);
            }
        }
    }
}

// -------------------------------------------------------------- locating --

struct Share {
    int n_eff;      // workgroups in use
    int s, e;       // flat page range of this workgroup
    int bg, base;   // first (sequence, kv head) touching s and its flat start
    int total;      // pages over all (sequence, kv head) pairs
    int q0, q1, lk; // pages_of's loaded words for pair bg (valid when bg < pairs)
};

// Work split (stream-K over pages).  The (sequence, kv head) pairs are laid
// end to end in page order; workgroup w takes an equal share of their cost.
// A pair costs its page count, plus piece_cost pages when its first page does
// not start a workgroup's share of an equal split by pages: such a workgroup
// then works on two pieces, and the extra piece's epilogue and prologue take
// about as long as piece_cost pages (with piece_cost = 0 the split is by pages
// alone).  The cost of a pair sits before its pages: a cost position x inside
// pair bg (cost range [C_bg, C_bg + cost_bg)) is page
//   base_bg + max(0, x - C_bg - (cost_bg - cnt_bg))
// of the flat page order, and workgroup w works on the pages between those of
// cost positions w T / n and (w + 1) T / n (T = total cost, n = workgroups).
// The merge kernel inverts the same mapping from ws_prefix and ws_cost.
//
// Every wave runs this (no LDS, no barrier): total page count, the number of
// workgroups in use, this workgroup's page range, and where it starts.
__device__ __forceinline__ bool starts_a_share(int base, int total, int n)
{
    // is base one of the page boundaries floor(w total / n), w = 0 .. n, of an
    // equal split?  With r = (base n) mod total that holds iff r == 0 or
    // r > total - n.  The quotient comes from a float estimate, corrected.
    const int64_t bn = (int64_t)base * n;
    int64_t w = (int64_t)((float)bn * __builtin_amdgcn_rcpf((float)total));
    int64_t r = bn - w * total;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (r < 0) {
            --w;
            r += total;
        }
        if (r >= total) {
            ++w;
            r -= total;
        }
    }
    return r == 0 || r > total - n;
}

__device__ Share locate(const SplitParams &p, int w, int lane, bool write_prefix)
{
    const int bh = p.num_seqs * p.hkv;
    const int C = p.piece_cost;
    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;   // lanes < this one
    Share sh;
    sh.s = sh.e = sh.base = 0;
    sh.q0 = sh.q1 = sh.lk = 0;
    sh.bg = bh;
    // One chunk of up to 64 pairs, lane = pair: page counts, their prefix, the
    // pairs whose start falls inside a share and the prefix of the costs; then
    // the pairs holding the cost positions cs and ce of this workgroup's share.
    // With at most 64 pairs everything comes from one load of the counts.
    auto chunk = [&](int c0, int cnt, int incl, int base, int cbase, int total, int n, int64_t cs, int64_t ce,
                     bool &found_s, bool &found_e, int rq0, int rq1, int rlk) {
        const int bg = c0 + lane;
        const int pb = base + incl - cnt;              // this lane's pair: first page
        const bool inside = C > 0 && bg < bh && bg > 0 && cnt > 0 && !starts_a_share(pb, total, n);
        const unsigned long long im = __ballot(inside);
        const int extra = inside ? C : 0;              // cost beyond the pages
        const int cb = cbase + (pb - base) + C * __builtin_popcountll(im & below);   // first cost position
        const int cend = cb + cnt + extra;
        if (write_prefix && bg < bh) {
            p.ws_prefix[bg] = pb;
            p.ws_cost[bg] = cb;
        }
        if (!found_s) {
            const unsigned long long hit = __ballot(bg < bh && cend > cs);
            if (hit) {
                const int ln = __ffsll((long long)hit) - 1;
                const int pg = pb + (int)max((int64_t)0, cs - cb - extra);
                sh.bg = c0 + ln;
                sh.base = __builtin_amdgcn_readlane(pb, ln);
                sh.s = __builtin_amdgcn_readlane(pg, ln);
                sh.q0 = __builtin_amdgcn_readlane(rq0, ln);
                sh.q1 = __builtin_amdgcn_readlane(rq1, ln);
                sh.lk = __builtin_amdgcn_readlane(rlk, ln);
                found_s = true;
            }
        }
        if (!found_e) {
            const unsigned long long hit = __ballot(bg < bh && cend > ce);
            if (hit) {
                const int ln = __ffsll((long long)hit) - 1;
                const int pg = pb + (int)max((int64_t)0, ce - cb - extra);
                sh.e = __builtin_amdgcn_readlane(pg, ln);
                found_e = true;
            }
        }
        return C * __builtin_popcountll(im);           // the chunk's cost beyond its pages
    };
    auto finish = [&](int total, int n, int64_t T) {
        if (write_prefix && lane == 0) {
            p.ws_prefix[bh] = total;
            p.ws_cost[bh] = (int)T;
            p.ws_meta[0] = n;
        }
    };
    if (bh <= 64) {
        int rq0 = 0, rq1 = 0, rlk = 0;
        const int cnt = lane < bh ? pages_of(p, lane, rq0, rq1, rlk) : 0;
        const int incl = wave_scan_dpp(cnt);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int n = min(p.grid_n, max(1, total / max(1, p.min_pages)));
        sh.n_eff = n;
        sh.total = total;
        const bool inside = C > 0 && lane < bh && lane > 0 && cnt > 0 && !starts_a_share(incl - cnt, total, n);
        const int64_t T = total + (int64_t)C * __builtin_popcountll(__ballot(inside));
        const int64_t cs = ((int64_t)w * T) / n, ce = ((int64_t)(w + 1) * T) / n;
        sh.s = sh.e = sh.base = total;
        bool found_s = false, found_e = false;
        chunk(0, cnt, incl, 0, 0, total, n, cs, ce, found_s, found_e, rq0, rq1, rlk);
        finish(total, n, T);
        return sh;
    }
    int total = 0;
    for (int c0 = 0; c0 < bh; c0 += 64) {
        const int bg = c0 + lane;
        total += __builtin_amdgcn_readlane(wave_scan_dpp(bg < bh ? pages_of(p, bg) : 0), 63);
    }
    const int n = min(p.grid_n, max(1, total / max(1, p.min_pages)));
    sh.n_eff = n;
    sh.total = total;
    int64_t T = total;
    if (C > 0) {
        int base = 0;
        for (int c0 = 0; c0 < bh; c0 += 64) {
            const int bg = c0 + lane;
            const int cnt = bg < bh ? pages_of(p, bg) : 0;
            const int incl = wave_scan_dpp(cnt);
            const bool inside = bg < bh && bg > 0 && cnt > 0 && !starts_a_share(base + incl - cnt, total, n);
            T += (int64_t)C * __builtin_popcountll(__ballot(inside));
            base += __builtin_amdgcn_readlane(incl, 63);
        }
    }
    const int64_t cs = ((int64_t)w * T) / n, ce = ((int64_t)(w + 1) * T) / n;
    sh.s = sh.e = sh.base = total;
    bool found_s = false, found_e = false;
    int base = 0, cbase = 0;
    for (int c0 = 0; c0 < bh; c0 += 64) {
        const int bg = c0 + lane;
        int rq0 = 0, rq1 = 0, rlk = 0;
        const int cnt = bg < bh ? pages_of(p, bg, rq0, rq1, rlk) : 0;
        const int incl = wave_scan_dpp(cnt);
        const int ctotal = __builtin_amdgcn_readlane(incl, 63);
        cbase += ctotal + chunk(c0, cnt, incl, base, cbase, total, n, cs, ce, found_s, found_e, rq0, rq1, rlk);
        base += ctotal;
        if (found_s && found_e && !write_prefix)
            break;
    }
    finish(total, n, T);
    return sh;
}

// ------------------------------------------------- FP8 kernel, LDS ring --

// Direct global -> LDS copy of 16 bytes per lane: global address sbase + voff
// (per lane), LDS address lds_addr + 16 * lane.  Issued as inline asm so the
// compiler does not insert a conservative wait for it before every LDS read;
// the ring below waits on vmcnt itself.  No other vector-memory instruction
// is issued inside the page loop, so the counts are exact.
// The copies carry the nontemporal hint (nt): every cache byte is read once
// per call, so nothing is gained by keeping its lines in L2 or the last-level
// cache, and with the hint the same calls run 3-10 % faster (measured on the
// long-context, high-concurrency, shape-sweep and MLA workloads, with four
// rotating copies of the pools so that no call finds the previous one's data).
// M0 is written inside the statement and listed as clobbered; nothing else in
// these kernels reads M0 (clang warns that it is a reserved register).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// The same copy from a per-lane 64-bit global address (key rows gathered one
// by one in the prefix + extend layout).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_at(const void *addr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(addr), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// Token-row gather, prefix + extend layout.  A "tag" names the row of one key:
// >= 0 a row of the k / v buffers, < 0 the row ~tag of kext / vext.  Each
// lane loads the kv_indices entry of one key of a step (unconditionally, from
// a clamped address, so the load can stay in flight: nothing reads the value
// until the step that issues the copies), and turns it into a tag there.
__device__ __forceinline__ int32_t tok_load(const SplitParams &p, int b, int s0, int pre, int j)
{
    const int32_t *a = pre > 0 ? p.kv_indices + s0 + min(max(j, 0), pre - 1) : p.kv_indptr + b;
    return *a;
}

__device__ __forceinline__ int32_t tok_tag(int32_t raw, int j, int pre, int lk, int q0, int64_t num_rows)
{
    if (j < pre)
        return raw < 0 ? 0 : (raw >= num_rows ? (int32_t)(num_rows - 1) : raw);
    return j < lk ? ~(q0 + (j - pre)) : 0;              // keys past lk are masked; row 0 is a safe read
}

__device__ __forceinline__ const uint8_t *tok_row(int32_t tag, const uint8_t *buf, const uint8_t *ext,
                                                  int64_t row_bytes)
{
    return tag >= 0 ? buf + (int64_t)tag * row_bytes : ext + (int64_t)(~tag) * row_bytes;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n that is a multiple of 8 in [0, 40]
// (a smaller n only waits longer).
__device__ __forceinline__ void wait_vmcnt_x8(int n)
{
    if (n >= 40)
        wait_vmcnt<40>();
    else if (n >= 32)
        wait_vmcnt<32>();
    else if (n >= 24)
        wait_vmcnt<24>();
    else if (n >= 16)
        wait_vmcnt<16>();
    else if (n >= 8)
        wait_vmcnt<8>();
    else
        wait_vmcnt<0>();
}

// One ring stage = one step (two pages) of one kv head, 16 KiB:
//   [K page a | K page b | V page a | V page b], 4 KiB each, 16 key rows of
//   256 bytes.  The 16-byte chunk c of key row n sits at slot c ^ n of the row
//   (XOR swizzle), so the operand reads below touch 16 distinct slots per 16 lanes.
constexpr int kStageBytes = 16384;
constexpr int kDmaPerPart = 8;           // copy instructions per wave and step (two 4 KiB pages)

// Lane offsets of the 4 copy instructions of one page: instruction i, lane l
// writes LDS bytes [1024 i + 16 l, +16) = key row n = 4i + l/16, slot l%16, so it
// fetches chunk (l%16) ^ n of that key row.  16 lanes read one 256-byte row.
__device__ __forceinline__ void dma_lane_offsets(uint32_t (&off)[4], int hkv, int lane)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = 4 * i + (lane >> 4);
        off[i] = (uint32_t)(n * hkv * kHeadDim + (((lane & 15) ^ n) * 16));
    }
}

// Half of a step copy: the K pages (part 0) or the V pages (part 1), 8
// instructions.  Two waves that share a ring stage issue one part each.
__device__ __forceinline__ void dma_step_part(uint32_t stage, const uint8_t *pool, int part, int64_t ya,
                                              int64_t yb, int64_t page_bytes, const uint32_t (&off)[4])
{
    const uint8_t *a = pool + ya * page_bytes;
    const uint8_t *b = pool + yb * page_bytes;
    const uint32_t base = stage + 8192 * part;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dma16(a, off[i], base + 1024 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dma16(b, off[i], base + 4096 + 1024 * i);
}

// ------------------------------------------- QK on fp8 (Q split hi + lo) --
//
// For the FP8 cache the QK^T contraction runs on v_mfma_f32_16x16x128_f8f6f4
// with K used as stored.  Each packed Q row r (bf16) is scaled by 2^k_r so its
// largest magnitude lies in [128, 256), then split into
//   hi = e4m3(q 2^k_r),  lo = e4m3(q 2^k_r - hi)   (round to nearest even).
// For every element of magnitude >= 2^-2 after scaling (all but those below
// 1/512 of the row maximum) hi + lo equals the scaled bf16 value exactly: the
// bits of a bf16 value below the top four fit one more e4m3 value.  Smaller
// elements are kept to 2^-10 absolute, i.e. 2^-17 of the row scale.  So
// S = K.hi + K.lo carries the same information as the bf16 product, and the
// logit multiplier of row r absorbs 2^-k_r.
//
// LDS layout of the Q operands: [rt][kc][part][half][lane] x 16 bytes, where
// kc selects dims [128 kc, 128 kc + 128), part 0 = hi, 1 = lo, and lane l
// holds row 16 rt + l%16, dims 128 kc + 32 (l/16) + 16 half .. +16.  Keeping a
// lane's two halves 1 KiB apart makes each 16-byte operand read of a wave one
// contiguous 1 KiB (a 32-byte lane stride costs a two-way bank conflict).
constexpr int kQf8Bytes = 4 * 2 * 2 * 64 * 32;              // up to 4 row tiles: 32 KiB

// The piece's packed Q rows arrive in the Q area as bf16, 512 B per row
// r = t G + h, by direct copies; the 16-byte chunk c of row r sits at slot
// c ^ (r & 15) so that the 16 rows read by one lane group hit 16 different
// banks.  Each wave reads the rows of its own row
// group in the order its lanes consume them: lane l takes row 16 (rg RTW + rt)
// + l%16 and dims 128 kc + 32 (l/16) .. +32 for kc = 0, 1.  The four lanes
// that share a row hold all 256 dims, so two lane exchanges give every lane
// its row's maximum and exponent k_r, which the lane keeps (the row's logit
// multiplier is c 2^-k_r).  After a barrier (every wave holds its rows) the
// four key groups of the row group overwrite the area with the fp8 operands,
// one (row tile, dim half) block each.
template <int RTW>
__device__ __forceinline__ void convert_q_block(unsigned char *qlds, const uint32_t (&raw)[16], int k, int blk,
                                                int lane)
{
    auto lo_f = [](uint32_t w) { return __builtin_bit_cast(float, w << 16); };
    auto hi_f = [](uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); };
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float s0 = ldexpf(lo_f(raw[2 * i]), k), s1 = ldexpf(hi_f(raw[2 * i]), k);
        const float s2 = ldexpf(lo_f(raw[2 * i + 1]), k), s3 = ldexpf(hi_f(raw[2 * i + 1]), k);
        int hw = __builtin_amdgcn_cvt_pk_fp8_f32(s0, s1, 0, false);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(s2, s3, hw, true);
        const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
        const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
        int lw = __builtin_amdgcn_cvt_pk_fp8_f32(s0 - h01[0], s1 - h01[1], 0, false);
        lw = __builtin_amdgcn_cvt_pk_fp8_f32(s2 - h23[0], s3 - h23[1], lw, true);
        hi[i] = (uint32_t)hw;
        lo[i] = (uint32_t)lw;
    }
    // block blk = rt * 2 + kc of the whole tile set; parts 0 (hi) and 1 (lo)
    uint4 *dh = reinterpret_cast<uint4 *>(qlds + (size_t)(blk * 2) * 2048 + lane * 16);
    uint4 *dl = reinterpret_cast<uint4 *>(qlds + (size_t)(blk * 2 + 1) * 2048 + lane * 16);
    dh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    dh[64] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    dl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    dl[64] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
}

template <int RTW>
__device__ __forceinline__ void stage_q_fp8(unsigned char *qlds, float (&crow)[RTW], float c,
                                            const SplitParams &p, int lq, int rg, int kg, int lane)
{
    const int j = lane >> 4;
    uint32_t raw[RTW][2][16];                              // bf16 pairs of dims 128 kc + 32 j ..
    int kx[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int n = lane & 15;
        const int r = (rg * RTW + rt) * 16 + n;             // packed row
        const bool live = (r >> p.log2g) < lq;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int chunk = 16 * kc + 4 * j + i;      // dims 8 chunk .. +8
                const uint4 q4 = live ? *reinterpret_cast<const uint4 *>(qlds + (size_t)r * 512 + ((chunk ^ n) * 16))
                                      : make_uint4(0, 0, 0, 0);
                raw[rt][kc][4 * i] = q4.x;
                raw[rt][kc][4 * i + 1] = q4.y;
                raw[rt][kc][4 * i + 2] = q4.z;
                raw[rt][kc][4 * i + 3] = q4.w;
            }
        }
    }
    auto lo_f = [](uint32_t w) { return __builtin_bit_cast(float, w << 16); };
    auto hi_f = [](uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); };
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        float amax = 0.f;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                amax = fmaxf(amax, fmaxf(fabsf(lo_f(raw[rt][kc][i])), fabsf(hi_f(raw[rt][kc][i]))));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));         // row max (4 lanes)
        int k = 0;
        if (amax > 0.f) {
            int e;
            frexpf(amax, &e);                              // amax in [2^(e-1), 2^e)
            k = min(8 - e, 127);
        }
        crow[rt] = ldexpf(c, -k);
        kx[rt] = k;
    }
    __syncthreads();                                       // every wave holds its rows
    // key group kg converts block (row tile kg / 2, dim half kg % 2)
    if (kg >= 2 * RTW)
        return;
    if (kg == 0)
        convert_q_block<RTW>(qlds, raw[0][0], kx[0], rg * RTW * 2 + 0, lane);
    else if (kg == 1)
        convert_q_block<RTW>(qlds, raw[0][1], kx[0], rg * RTW * 2 + 1, lane);
    if constexpr (RTW == 2) {
        if (kg == 2)
            convert_q_block<RTW>(qlds, raw[1][0], kx[1], rg * RTW * 2 + 2, lane);
        else if (kg == 3)
            convert_q_block<RTW>(qlds, raw[1][1], kx[1], rg * RTW * 2 + 3, lane);
    }
}

// QK^T of a step (two pages) on fp8: S^T[a][rt] (16 keys x 16 rows) from the
// ring stage's K rows and the staged hi/lo Q operands.  K operand: lane (n =
// l%16, j = l/16) holds dims 128 kc + 32 j .. +32 of key n, i.e. 16-byte chunks
// 8 kc + 2 j and 8 kc + 2 j + 1 (stored at slots chunk ^ n).
template <int RTW>
__device__ __forceinline__ void qk_lds_f8(floatx4_t (&S)[2][RTW], const unsigned char *stage,
                                          const unsigned char *qw, int lane)
{
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
            S[a][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        intx8_t kop[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int c0 = 8 * kc + 2 * j;
            const uint4 lo4 = *reinterpret_cast<const uint4 *>(stage + 4096 * a + 256 * n + 16 * (c0 ^ n));
            const uint4 hi4 = *reinterpret_cast<const uint4 *>(stage + 4096 * a + 256 * n + 16 * ((c0 + 1) ^ n));
            kop[a] = intx8_t{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                             (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
        }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const uint4 *qp = reinterpret_cast<const uint4 *>(
                    qw + (size_t)((rt * 2 + kc) * 2 + part) * 2048 + lane * 16);
                const uint4 b0 = qp[0], b1 = qp[64];
                const intx8_t qop = intx8_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    S[a][rt] = mfma16_f8(kop[a], qop, S[a][rt]);
            }
    }
}

// ------------------------------------------------------- piece epilogue --
//
// The 4 key groups of a row group hold softmax states (m, l, O) of the same
// rows over disjoint keys.  Each wave publishes per row its m and l and its
// normalised O/l in fp16 (|O/l| <= max |V| <= 448 for an e4m3 cache, so fp16
// keeps 11 significant bits), then all 512 threads combine the four states
// in fp32, one (row, 8-dim chunk) per thread, and store 16 contiguous bytes:
// bf16 output when the piece is the whole (sequence, kv head), else the
// piece's partial (fp16 O/L and the fp32 log2-domain LSE) for the reduce.
//
// LDS after the page loop: [0, 2 KiB) holds m, l of [kg][row]; the ring area
// holds [kg][row] rows of 256 fp16 whose 16-byte chunk c sits at c ^ (row & 15)
// (writes from the accumulator layout and row-wise reads are both free of
// bank conflicts).

// The thread index, hidden from loop-invariant code motion: address math of
// the per-piece epilogue would otherwise be hoisted above the page loop and
// hold registers (spilled) through it.
__device__ __forceinline__ int opaque_tid()
{
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const half2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}

__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Key-group exchange format of the epilogue: fp16 (FP8 cache) or bf16 (bf16 cache).
template <int KVT>
__device__ __forceinline__ uint32_t xpack(float a, float b)
{
    if constexpr (KVT == kKvFp8)
        return pack_f16x2(a, b);
    else
        return pack_bf16x2(a, b);
}

template <int KVT>
__device__ __forceinline__ float xlo(uint32_t w)
{
    if constexpr (KVT == kKvFp8)
        return f16_lo(w);
    else
        return __builtin_bit_cast(float, w << 16);
}

template <int KVT>
__device__ __forceinline__ float xhi(uint32_t w)
{
    if constexpr (KVT == kKvFp8)
        return f16_hi(w);
    else
        return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

template <int RTW, int KVT>
__device__ __forceinline__ void piece_epilogue(RowState<RTW> &st, unsigned char *lds, unsigned char *obuf,
                                               const SplitParams &p, int kg, int rg, int lane, int lq,
                                               int q0, int g, int slot, bool whole, float vd)
{
    constexpr int NG = 4;
    constexpr int RT = 2 * RTW;                          // row tiles of the workgroup
    const int G = 1 << p.log2g;
    const int n = lane & 15, j = lane >> 4;
    float *ml = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        float t = st.l[rt];
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        st.l[rt] = t;
    }
    __syncthreads();                                     // every wave is past the page loop
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int row = (rg * RTW + rt) * 16 + n;
        if (j == 0) {
            ml[(kg * 64 + row) * 2] = st.m[rt];
            ml[(kg * 64 + row) * 2 + 1] = st.l[rt];
        }
        const float inv = st.l[rt] > 0.f ? 1.0f / st.l[rt] : 0.f;
        unsigned char *orow = obuf + (size_t)(kg * 64 + row) * 512;
#pragma unroll
        for (int e = 0; e < 4; ++e) {                    // dims 64 j + 16 e + t, t = 0..15
            uint4 a, b;
            a.x = xpack<KVT>(st.o[0][rt][e] * inv, st.o[1][rt][e] * inv);
            a.y = xpack<KVT>(st.o[2][rt][e] * inv, st.o[3][rt][e] * inv);
            a.z = xpack<KVT>(st.o[4][rt][e] * inv, st.o[5][rt][e] * inv);
            a.w = xpack<KVT>(st.o[6][rt][e] * inv, st.o[7][rt][e] * inv);
            b.x = xpack<KVT>(st.o[8][rt][e] * inv, st.o[9][rt][e] * inv);
            b.y = xpack<KVT>(st.o[10][rt][e] * inv, st.o[11][rt][e] * inv);
            b.z = xpack<KVT>(st.o[12][rt][e] * inv, st.o[13][rt][e] * inv);
            b.w = xpack<KVT>(st.o[14][rt][e] * inv, st.o[15][rt][e] * inv);
            const int c0 = 8 * j + 2 * e;
            *reinterpret_cast<uint4 *>(orow + ((c0 ^ n) * 16)) = a;
            *reinterpret_cast<uint4 *>(orow + (((c0 + 1) ^ n) * 16)) = b;
        }
    }
    __syncthreads();
    const int tid = opaque_tid();
    const int c = tid & 31;
    const int nrows = min(lq * G, RT * 16);
    for (int r = tid >> 5; r < nrows; r += 16) {
        float mk[NG], lk[NG];
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            mk[k] = ml[(k * 64 + r) * 2];
            lk[k] = ml[(k * 64 + r) * 2 + 1];
            M = fmaxf(M, lk[k] > 0.f ? mk[k] : -INFINITY);
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float W = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const float w = lk[k] > 0.f ? lk[k] * exp2_fast(mk[k] - M) : 0.f;
            W += w;
            const uint4 v = *reinterpret_cast<const uint4 *>(obuf + (size_t)(k * 64 + r) * 512 +
                                                             ((c ^ (r & 15)) * 16));
            acc[0] += w * xlo<KVT>(v.x);
            acc[1] += w * xhi<KVT>(v.x);
            acc[2] += w * xlo<KVT>(v.y);
            acc[3] += w * xhi<KVT>(v.y);
            acc[4] += w * xlo<KVT>(v.z);
            acc[5] += w * xhi<KVT>(v.z);
            acc[6] += w * xlo<KVT>(v.w);
            acc[7] += w * xhi<KVT>(v.w);
        }
        const int t = r >> p.log2g, h = r & (G - 1);
        if (whole) {
            if (p.sinks) {                               // the sink joins the denominator only
                const float sk = p.sinks[g * G + h] * 1.4426950408889634f;
                const float mm = fmaxf(M, sk);
                const float f = W > 0.f ? exp2_fast(M - mm) : 0.f;
                W = W * f + exp2_fast(sk - mm);
#pragma unroll
                for (int d = 0; d < 8; ++d)
                    acc[d] *= f;
            }
            const float sc = W > 0.f ? vd / W : 0.f;
            uint4 o;
            o.x = pack_bf16x2(acc[0] * sc, acc[1] * sc);
            o.y = pack_bf16x2(acc[2] * sc, acc[3] * sc);
            o.z = pack_bf16x2(acc[4] * sc, acc[5] * sc);
            o.w = pack_bf16x2(acc[6] * sc, acc[7] * sc);
            *reinterpret_cast<uint4 *>(p.out + ((int64_t)(q0 + t) * p.hq + g * G + h) * kHeadDim + 8 * c) = o;
        } else {
            const float sc = W > 0.f ? 1.0f / W : 0.f;
            const int64_t sr = ((int64_t)slot * p.rows_max + r) * kHeadDim + 8 * c;
            if constexpr (KVT == kKvFp8) {                  // fp16 partial: |O/l| <= 448
                uint4 o;
                o.x = pack_f16x2(acc[0] * sc, acc[1] * sc);
                o.y = pack_f16x2(acc[2] * sc, acc[3] * sc);
                o.z = pack_f16x2(acc[4] * sc, acc[5] * sc);
                o.w = pack_f16x2(acc[6] * sc, acc[7] * sc);
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.ws_o) + sr) = o;
            } else {                                        // fp32 partial: any bf16 V
                float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(p.ws_o) + sr);
                dst[0] = make_float4(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc);
                dst[1] = make_float4(acc[4] * sc, acc[5] * sc, acc[6] * sc, acc[7] * sc);
            }
            if (c == 0)
                p.ws_lse[(int64_t)slot * p.rows_max + r] = W > 0.f ? M + __log2f(W) : -INFINITY;
        }
    }
}

// FP8 split-KV kernel, 8 waves (two per SIMD, so one wave's MFMA work runs
// while the other's vector work issues).  The waves form 4 key groups x 2 row
// groups: a wave holds RTW row tiles (row group rg) and computes every 4th
// step (page pair) of the piece (key group kg).  The two waves of a key group
// share a 2-stage LDS ring: for each step one copies the K pages and the other
// the V pages, straight from HBM, one step ahead of the compute.  One
// workgroup barrier per step makes a stage visible to both waves and frees the
// stage the next copy overwrites.
template <int RTW, bool CAP, bool TOK>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void va_split_kv_fp8_w8_kernel(SplitParams p)
{
    constexpr int NG = 4;
    constexpr int kQBytes = kQf8Bytes;                      // fp8 hi/lo Q operands, 4 row tiles
    constexpr int kRingBytes = 2 * kStageBytes;              // per key group
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kQBytes + NG * kRingBytes];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int rg = wave & 1;
    const int kg = wave >> 1;
    const int w = blockIdx.x;
    const int G = 1 << p.log2g;

    Share sh = locate(p, w, lane, w == 0 && wave == 0);
    sh.n_eff = uniform(sh.n_eff);
    sh.s = uniform(sh.s);
    sh.e = uniform(sh.e);
    sh.bg = uniform(sh.bg);
    sh.base = uniform(sh.base);
    if (w >= sh.n_eff)
        return;                                        // uniform over the workgroup

    const float kd = load_descale(p.kdesc);
    const float vd = load_descale(p.vdesc);
    const float c = p.scale_log2 * kd;
    unsigned char *ring = lds + kQBytes + kg * kRingBytes;
    const uint32_t ring_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(ring));
    const unsigned char *qw = lds + (size_t)rg * RTW * 2 * 2 * 64 * 32;
    const int64_t page_bytes = (int64_t)kPage * p.hkv * kHeadDim;

    const int bh = p.num_seqs * p.hkv;
    int s = sh.s, bg = sh.bg, base = sh.base;
    while (s < sh.e && bg < bh) {
        // Per-lane values are rederived for each piece from an opaque lane
        // index, so their address math is not hoisted above the piece loop
        // (it would hold registers through the page loop and be spilled).
        int pl = lane;
        asm volatile("" : "+v"(pl));
        uint32_t off[4];
        dma_lane_offsets(off, p.hkv, pl);
        const int b = uniform(bg / p.hkv);
        const int g = bg - b * p.hkv;
        const int q0 = load_uniform(p.cu, b);
        const int lq = checked_q_len(q0, load_uniform(p.cu, b + 1), p.total_q, p.max_q);
        int s0 = 0, lk;                                        // s0: prefix start in kv_indices
        if constexpr (TOK) {
            s0 = load_uniform(p.kv_indptr, b);
            lk = prefix_keys(s0, load_uniform(p.kv_indptr, b + 1), lq, p.num_indices);
        } else {
            lk = load_uniform(p.seqused, b);
        }
        const int pb = first_page(lk, lq, p.window_left);      // the range starts at logical page pb
        const int cnt = (lq <= 0 || lk <= 0) ? 0 : max(0, min((lk + kPage - 1) / kPage, p.mbps) - pb);
        if (cnt == 0) {
            ++bg;
            continue;
        }
        const int ctx = lk - lq;
        const int r0 = s - base;                               // piece = pages r0 .. r1 of the pair's range
        const int r1 = min(sh.e, base + cnt) - base;
        const bool whole = (r0 == 0 && r1 == cnt);
        const int p0 = pb + r0, p1 = pb + r1;
        const int slot = 2 * w + (s != sh.s);           // first or last piece of this workgroup
        const int lo_max = p.window_left < 0 ? INT_MIN : ctx + lq - 1 - p.window_left;
        const uint32_t wlim = p.window_left < 0 ? 0x7FFFFFFFu : (uint32_t)p.window_left;

        const int npairs = (p1 - p0 + 1) >> 1;
        const int nsteps = (npairs + NG - 1) / NG;             // uniform over the workgroup
        const bool rows_live = (rg * RTW * 16) < lq * G;
        const int32_t *btrow = p.bt + (int64_t)b * p.mbps;
        const uint8_t *pool = (rg == 0 ? p.k : p.v) + (int64_t)g * kHeadDim;
        const int64_t maxpage = p.num_blocks - 1;
        auto phys = [&](int page) -> int64_t {
            int64_t v = load_uniform(btrow, uniform(page));
            v = v < 0 ? 0 : v;
            return v > maxpage ? maxpage : v;
        };
        auto issue = [&](int k, int stage) {                   // this wave's half of step k
            const int pa = p0 + 2 * k;
            const int64_t ya = phys(pa);
            const int64_t yb = pa + 1 < p1 ? phys(pa + 1) : ya;
            dma_step_part(ring_addr + stage * kStageBytes, pool, rg, ya, yb, page_bytes, off);
        };
        // prefix + extend layout: lane l tags key 32 k' + l % 32 of step k
        // (k' = the step's first key / 32); copy i of the wave takes key row
        // n = 4 (i % 4) + l / 16 of page i / 4, chunk (l % 16) ^ n, as above.
        const int pre = lk - lq;
        const uint8_t *ext = (rg == 0 ? p.kext : p.vext) + (int64_t)g * kHeadDim;
        const int64_t row_bytes = (int64_t)p.hkv * kHeadDim;
        auto tload = [&](int k) { return tok_load(p, b, s0, pre, (p0 + 2 * k) * kPage + (pl & 31)); };
        auto issue_tok = [&](int k, int stage, int32_t raw) {
            const int32_t tag = tok_tag(raw, (p0 + 2 * k) * kPage + (pl & 31), pre, lk, q0, p.num_rows);
            const uint32_t dst = ring_addr + stage * kStageBytes + 8192 * rg;
            int32_t t[8];                                      // all shuffles first: one LDS round trip
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t[i] = __shfl(tag, 16 * (i >> 2) + 4 * (i & 3) + (pl >> 4));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int n = 4 * (i & 3) + (pl >> 4);
                dma16_at(tok_row(t[i], pool, ext, row_bytes) + (((pl & 15) ^ n) * 16),
                         dst + 4096 * (i >> 2) + 1024 * (i & 3));
            }
        };
        // The tags of the first two steps are read before any copy is issued;
        // later ones one step ahead (rawN), so each is in registers when its
        // step's copies go out.  Nothing reads a tag load's register before
        // the wait that covers it (the empty asm statements mark those points).
        int32_t rawA = 0, rawB = 0, rawN = 0;
        if constexpr (TOK) {
            rawA = tload(kg);
            rawB = tload(kg + NG);
            asm volatile("" : "+v"(rawA), "+v"(rawB));
        }

        // ---- prologue: Q rows and the first step's pages are copied
        // straight into LDS; the Q conversion overlaps the page copies.  The
        // second step is issued only after the conversion: at the start of
        // the kernel every workgroup's first requests queue at once, and
        // requests for step 1 issued with them would share the bandwidth with
        // step 0 and delay it.
        __syncthreads();                                // previous piece's LDS reads done
        const uint32_t lds_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(lds));
        for (int i = wave; i < ((lq * G) >> 1); i += NG * 2) {        // row pairs: 1 KiB each
            const int r = 2 * i;                               // rows r, r + 1 share a token (G even)
            const int64_t row0 = uniform((int)((int64_t)(q0 + (r >> p.log2g)) * p.hq + g * G + (r & (G - 1))));
            const int rr = r + (pl >> 5), slot = pl & 31;      // lane's LDS row and slot
            dma16(p.q + row0 * kHeadDim, (uint32_t)((pl >> 5) * 512 + ((slot ^ (rr & 15)) * 16)), lds_addr + r * 512);
        }
        const bool has1 = kg + NG < npairs;
        if (kg < npairs) {
            if constexpr (TOK)
                issue_tok(kg, 0, rawA);
            else
                issue(kg, 0);
            wait_vmcnt<kDmaPerPart>();                  // this wave's Q copies landed
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();                                // every wave's Q copies landed
        float crow[RTW];                                       // logit multiplier of this lane's row
        stage_q_fp8<RTW>(lds, crow, c, p, lq, rg, kg, pl);
        if (has1) {
            if constexpr (TOK) {
                issue_tok(kg + NG, 1, rawB);
                rawN = tload(kg + 2 * NG);
            } else {
                issue(kg + NG, 1);
            }
        }

        RowState<RTW> st;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            st.m[rt] = -INFINITY;
            st.l[rt] = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t)
                st.o[t][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
        int limit[RTW];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const int t = ((rg * RTW + rt) * 16 + (pl & 15)) >> p.log2g;
            limit[rt] = min(ctx + t, lk - 1);
        }


        for (int t = 0; t < nsteps; ++t) {
            const int k = kg + t * NG;
            if (t == 0 && k + NG < npairs)                     // own copies of step 0 landed (step 1 may
                wait_vmcnt<TOK ? kDmaPerPart + 1 : kDmaPerPart>();   // not, nor step 2's tags)
            else
                wait_vmcnt<0>();                               // own copies of step t landed
            if constexpr (TOK) {
                if (t >= 1)
                    asm volatile("" : "+v"(rawN));             // step t+1's tags: loaded with step t
            }
            __syncthreads();                                   // partner's too; stage of step t-1 is free

            if (t >= 1 && k + NG < npairs) {                   // steps 0 and 1 came with the prologue
                if constexpr (TOK) {
                    issue_tok(k + NG, (t + 1) & 1, rawN);
                    rawN = tload(k + 2 * NG);
                } else {
                    issue(k + NG, (t + 1) & 1);
                }
            }
            if (k < npairs && rows_live) {
                const unsigned char *stage = ring + (t & 1) * kStageBytes;
                floatx4_t S[2][RTW];
                qk_lds_f8<RTW>(S, stage, qw, pl);
                const int pa = p0 + 2 * k;
                const bool hb = pa + 1 < p1;
                const int key0 = pa * kPage;
                const bool masked = !hb || key0 + 31 > ctx || key0 < lo_max;
                bf16x8_t pop[RTW];
                softmax_step<RTW, CAP>(st, pop, S, limit, wlim, key0, hb, crow, p.cap_log2, pl, masked);
                pv_lds<RTW>(st, stage, pop, masked, masked ? v_zero_mask(key0, hb, lk, pl) : 0u, pl);
            }
        }
        wait_vmcnt<0>();

        piece_epilogue<RTW, kKvFp8>(st, lds, lds + kQBytes, p, kg, rg, pl, lq, q0, g, slot, whole, vd);


        s = base + r1;
        base += cnt;
        ++bg;
    }
}

// ------------------------------------ FP8 kernel, one wave per SIMD (w4) --
//
// 4 waves, one per SIMD.  Wave kg is key group kg: it computes every 4th step
// (page pair) of the piece for every packed row of the piece (RT row tiles,
// up to 64 rows), so each K and V byte a workgroup copies into LDS is read
// once and each V element is converted to bf16 once.  A wave's O^T
// accumulators (16 dim tiles x RT row tiles x 4 floats: 256 at RT = 4) sit in
// the accumulation registers; its fp8 hi / lo Q operands (32 registers per
// row tile) stay in vector registers for the whole piece, so the page loop
// reads only K and V from LDS.
//
// Each wave owns 40 KiB of LDS: a K ring of 6 page slots and a V ring of 4
// (4 KiB each: 16 key rows of 256 bytes; in K the 16-byte chunk c of row n
// sits at slot c ^ n, so the 16 rows a QK read touches fall in different
// banks; V rows are unswizzled, see w4_pv).  It copies its own pages into them and waits for them with vmcnt
// alone: no workgroup barrier inside the page loop, so the four waves run
// their steps independently.  Step t computes the wave's local pages 2t and
// 2t + 1 and refills its own slots as soon as it has read them: K of step
// t + 3 once its K reads have returned, V of step t + 2 once its V reads have.
// K therefore arrives about three steps ahead of its QK and V two steps ahead
// of its PV (one step of lead was less than the memory latency of a loaded GPU).
//
// Prologue of a piece: wave kg copies the bf16 rows of row tile kg into K
// slots 4 and 5, converts them in place into the hi / lo operands, and puts
// the rows' logit multipliers into the last KiB of V slot 3; after a barrier
// every wave loads all row tiles' operands into registers; after a second
// barrier (every wave holds them) those slots are handed back to the rings.
// The copies of steps 0 and 1 (all but that last KiB) go out with the Q rows,
// so only K of step 2 and one KiB of V wait for the exchange: the memory
// system has about 40 KiB per wave to fetch while the rows are converted.
// Epilogue: each wave writes its rows' m, l and scaled O (fp16) into its own
// 40 KiB (see w4_epilogue); after barriers all 256 threads combine them.
constexpr int kW4KSlots = 6;
constexpr int kW4VSlots = 4;
constexpr int kW4PageBytes = 4096;                          // one page of one kv head, K or V
constexpr int kW4VBase = kW4KSlots * kW4PageBytes;           // V ring offset in a wave's region
constexpr int kW4RingBytes = (kW4KSlots + kW4VSlots) * kW4PageBytes;   // 40 KiB per wave, 160 KiB in all
constexpr int kW4QStage = 4 * kW4PageBytes;                  // prologue: row tile (K slots 4, 5)
constexpr int kW4CStage = kW4VBase + 3 * kW4PageBytes + 3072; // prologue: row multipliers (V slot 3, last KiB)
constexpr int kW4Ml = 8 * kW4PageBytes;                      // epilogue: (m, l) of the rows (V slot 2)
constexpr int kW4Mw = kW4Ml + 512;                           // epilogue: (M, W) of the rows (wave 0)

// QK^T of a step on fp8 from register-resident Q operands: K page a at ka,
// page b at kb (slots of the ring).  qop[rt][kc][part]: row tile rt, dims
// [128 kc, 128 kc + 128), part 0 = hi, 1 = lo (lane layout as qk_lds_f8).
//
// The MFMAs are written as inline assembly so that their results stay in
// vector registers: with one wave per SIMD the compiler gives every MFMA an
// accumulation-register destination, and the 256 O^T accumulators already fill
// that file.  The compiler's hazard checks do not look inside the statements,
// so they carry the required gaps themselves:
//   - each statement starts with "s_nop 1": a vector ALU write of an operand
//     needs 2 wait states before an MFMA reads it;
//   - a chain accumulates into exactly its own registers, which same-shape
//     MFMAs may do back to back, and 2 RT - 1 other MFMAs separate them;
//   - w4_qk_done follows the last MFMA and every read of S depends on it: 19
//     wait states, where an MFMA of this shape (8 passes) needs 11 before
//     another instruction reads or writes its result.
// One group of a step's QK MFMAs: dims [128 kc, 128 kc + 128), part 0 (hi) or
// 1 (lo) of Q, all 2 RT chains (S[a][rt]: page a, row tile rt).  The first
// group starts the chains from zero.  Operands: S first (a-major), then the two
// K operands, then the RT Q operands.
template <int RT> struct W4QkGroup;
template <> struct W4QkGroup<1> {
    __device__ static __forceinline__ void first(floatx4_t (&S)[2][1], const intx8_t (&k)[2],
                                                 const intx8_t (&q)[1])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %2, %4, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %3, %4, 0\n\t"
            : "=&v"(S[0][0]), "=&v"(S[1][0])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]));
    }
    __device__ static __forceinline__ void acc(floatx4_t (&S)[2][1], const intx8_t (&k)[2],
                                               const intx8_t (&q)[1])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %2, %4, %0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %3, %4, %1\n\t"
            : "+v"(S[0][0]), "+v"(S[1][0])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]));
    }
};
template <> struct W4QkGroup<2> {
    __device__ static __forceinline__ void first(floatx4_t (&S)[2][2], const intx8_t (&k)[2],
                                                 const intx8_t (&q)[2])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %4, %6, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %2, %5, %6, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %4, %7, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %3, %5, %7, 0\n\t"
            : "=&v"(S[0][0]), "=&v"(S[0][1]), "=&v"(S[1][0]), "=&v"(S[1][1])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]));
    }
    __device__ static __forceinline__ void acc(floatx4_t (&S)[2][2], const intx8_t (&k)[2],
                                               const intx8_t (&q)[2])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %4, %6, %0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %2, %5, %6, %2\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %4, %7, %1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %3, %5, %7, %3\n\t"
            : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[1][0]), "+v"(S[1][1])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]));
    }
};
template <> struct W4QkGroup<3> {
    __device__ static __forceinline__ void first(floatx4_t (&S)[2][3], const intx8_t (&k)[2],
                                                 const intx8_t (&q)[3])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %6, %8, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %3, %7, %8, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %6, %9, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %4, %7, %9, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %2, %6, %10, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %5, %7, %10, 0\n\t"
            : "=&v"(S[0][0]), "=&v"(S[0][1]), "=&v"(S[0][2]), "=&v"(S[1][0]), "=&v"(S[1][1]), "=&v"(S[1][2])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]), "v"(q[2]));
    }
    __device__ static __forceinline__ void acc(floatx4_t (&S)[2][3], const intx8_t (&k)[2],
                                               const intx8_t (&q)[3])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %6, %8, %0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %3, %7, %8, %3\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %6, %9, %1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %4, %7, %9, %4\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %2, %6, %10, %2\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %5, %7, %10, %5\n\t"
            : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[0][2]), "+v"(S[1][0]), "+v"(S[1][1]), "+v"(S[1][2])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]), "v"(q[2]));
    }
};
template <> struct W4QkGroup<4> {
    __device__ static __forceinline__ void first(floatx4_t (&S)[2][4], const intx8_t (&k)[2],
                                                 const intx8_t (&q)[4])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %8, %10, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %4, %9, %10, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %8, %11, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %5, %9, %11, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %2, %8, %12, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %6, %9, %12, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %3, %8, %13, 0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %7, %9, %13, 0\n\t"
            : "=&v"(S[0][0]), "=&v"(S[0][1]), "=&v"(S[0][2]), "=&v"(S[0][3]), "=&v"(S[1][0]), "=&v"(S[1][1]), "=&v"(S[1][2]), "=&v"(S[1][3])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]));
    }
    __device__ static __forceinline__ void acc(floatx4_t (&S)[2][4], const intx8_t (&k)[2],
                                               const intx8_t (&q)[4])
    {
        asm("s_nop 1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %0, %8, %10, %0\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %4, %9, %10, %4\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %1, %8, %11, %1\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %5, %9, %11, %5\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %2, %8, %12, %2\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %6, %9, %12, %6\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %3, %8, %13, %3\n\t"
                "v_mfma_f32_16x16x128_f8f6f4 %7, %9, %13, %7\n\t"
            : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[0][2]), "+v"(S[0][3]), "+v"(S[1][0]), "+v"(S[1][1]), "+v"(S[1][2]), "+v"(S[1][3])
            : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]));
    }
};

template <int RT>
__device__ __forceinline__ void w4_qk_done(floatx4_t (&S)[2][RT])
{
    if constexpr (RT == 1)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(S[0][0]), "+v"(S[1][0]));
    else if constexpr (RT == 2)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
                     : "+v"(S[0][0]), "+v"(S[1][0]), "+v"(S[0][1]), "+v"(S[1][1]));
    else if constexpr (RT == 3)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
                     : "+v"(S[0][0]), "+v"(S[1][0]), "+v"(S[0][1]), "+v"(S[1][1]), "+v"(S[0][2]), "+v"(S[1][2]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
                     : "+v"(S[0][0]), "+v"(S[1][0]), "+v"(S[0][1]), "+v"(S[1][1]), "+v"(S[0][2]), "+v"(S[1][2]),
                       "+v"(S[0][3]), "+v"(S[1][3]));
}

template <int RT>
__device__ __forceinline__ void w4_qk(floatx4_t (&S)[2][RT], const unsigned char *ka, const unsigned char *kb,
                                      const intx8_t (&qop)[RT][2][2], int lane)
{
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        intx8_t kop[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const unsigned char *kp = a ? kb : ka;
            const int c0 = 8 * kc + 2 * j;
            const uint4 lo4 = *reinterpret_cast<const uint4 *>(kp + 256 * n + 16 * (c0 ^ n));
            const uint4 hi4 = *reinterpret_cast<const uint4 *>(kp + 256 * n + 16 * ((c0 + 1) ^ n));
            kop[a] = intx8_t{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                             (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
        }
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            intx8_t q[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                q[rt] = qop[rt][kc][part];
            if (kc == 0 && part == 0)
                W4QkGroup<RT>::first(S, kop, q);
            else
                W4QkGroup<RT>::acc(S, kop, q);
        }
    }
    w4_qk_done<RT>(S);
}

// Softmax part of a w4 step.  The accumulators are never rescaled inside the
// page loop: each row keeps a reference m (log2 units), set from its first
// visible keys, and p = 2^(x - m) is accumulated as long as x <= m + kTauW4.
// Then p <= 2^64, |p v| <= 2^73 for any e4m3 value, and fp32 sums of up to
// 2^24 keys stay below 2^97: no overflow, and the final O / l does not depend
// on m.  A step whose row maximum t exceeds m + kTauW4 sets `retry` and moves
// m to t; the rest of that pass is discarded, and the caller runs the piece's
// page loop again from the final m.  Every logit of the piece is then at most
// m + kTauW4 (steps that did not move m were within kTauW4 of an m that only
// grew; the others are at most the final m), so the second pass never moves
// m.  The row limit (last visible key) is derived only on masked steps.
// Other arguments as softmax_step.
constexpr float kTauW4 = 64.0f;

template <int RT, bool CAP, bool MASKED>
__device__ __forceinline__ void w4_softmax(RowState<RT> &st, bool &retry, bf16x8_t (&pop)[RT],
                                           const floatx4_t (&S)[2][RT], int ctx, int lk, int log2g,
                                           uint32_t wlim, int key0, bool has_b, const float (&c)[RT], float cap,
                                           int lane)
{
    const int j = lane >> 4;
    // ok[rt][i]: key i of this lane is visible to row (lane % 16) of tile rt
    auto visible = [&](int rt, int a, int e) {
        // last key row (lane % 16) of tile rt may see; a window starts wlim keys before it
        const int limit = min(ctx + ((16 * rt + (lane & 15)) >> log2g), lk - 1);
        const int key = key0 + 16 * a + 4 * j + e;
        return (a == 0 || has_b) && (uint32_t)(limit - key) <= wlim;
    };
    // Without a softcap the multiplier c >= 0 (a negative one is folded into
    // the sign of Q) only scales the logits: the row maximum is c max(S), and
    // p = 2^(S c - m) is one fma and one exp2.  With a softcap the capped
    // logits x are formed first.
    float x[RT][8];
    bool need_any = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = S[a][rt][e];
                if constexpr (CAP)
                    v = softcap_log2(v * c[rt], cap);
                if constexpr (MASKED)
                    v = visible(rt, a, e) ? v : -INFINITY;
                x[rt][4 * a + e] = v;
            }
        float lmax = fmaxf(fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3])),
                           fmaxf(fmaxf(x[rt][4], x[rt][5]), fmaxf(x[rt][6], x[rt][7])));
        if constexpr (!CAP)
            lmax = lmax == -INFINITY ? -INFINITY : lmax * c[rt];
        need_any |= lmax > st.m[rt] + kTauW4;                 // also a row's first visible keys
    }
    if (__any(need_any)) {                                     // rare: never touches O
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float t = x[rt][0];
#pragma unroll
            for (int i = 1; i < 8; ++i)
                t = fmaxf(t, x[rt][i]);
            if constexpr (!CAP)
                t = t == -INFINITY ? -INFINITY : t * c[rt];
            t = row4_max(t);                                  // row max of this step
            if (t > st.m[rt] + kTauW4) {
                retry |= st.m[rt] != -INFINITY;                // else nothing is accumulated yet
                st.m[rt] = t;
            }
        }
    }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float mref = st.m[rt] == -INFINITY ? 0.0f : st.m[rt];
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (CAP)
                p[i] = exp2_fast(x[rt][i] - mref);
            else if constexpr (MASKED)                         // a masked key is -inf, even when c = 0
                p[i] = x[rt][i] == -INFINITY ? 0.f : exp2_fast(__builtin_fmaf(x[rt][i], c[rt], -mref));
            else
                p[i] = exp2_fast(__builtin_fmaf(x[rt][i], c[rt], -mref));
        }
        uint4 w;
        w.x = pack_bf16x2(p[0], p[1]);
        w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]);
        w.w = pack_bf16x2(p[6], p[7]);
        // l sums the bf16 weights the PV MFMA uses
        float l = st.l[rt];
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), ones, l, false);
        st.l[rt] = l;
        pop[rt] = __builtin_bit_cast(bf16x8_t, w);
    }
}

// QK^T and softmax of an unmasked step without a softcap, with the row tiles
// pipelined: the MFMAs of row tile rt are issued between the vector
// instructions of row tile rt - 1's softmax, so that with one wave per SIMD the
// matrix unit and the vector unit work at the same time (in program order a
// run of MFMAs would hold the wave until the last one issues).  The softmax is
// computed optimistically from the current reference m: every p and l is what
// w4_softmax would produce unless some logit of the step exceeds m + kTauW4.
// That is tested per lane on the way; if any lane finds it, the l of the step
// is rolled back and w4_softmax redoes the step (it moves m and sets `retry`),
// so the result is w4_softmax's in every case.  The first step of a pass is
// such a case for each row (m starts at -inf).
//
// One pair of QK MFMAs (the two key pages of the step) of one (kc, part) group
// of row tile rt.  Same hazard handling as W4QkGroup; w4_qk_pad gives the 19
// wait states after the last pair of a row tile, before its S is read.
__device__ __forceinline__ void w4_qk_pair_first(floatx4_t &s0, floatx4_t &s1, const intx8_t &k0,
                                                 const intx8_t &k1, const intx8_t &q)
{
    asm volatile("s_nop 1\n\t"
                 "v_mfma_f32_16x16x128_f8f6f4 %0, %2, %4, 0\n\t"
                 "v_mfma_f32_16x16x128_f8f6f4 %1, %3, %4, 0"
                 : "=&v"(s0), "=&v"(s1)
                 : "v"(k0), "v"(k1), "v"(q));
}

__device__ __forceinline__ void w4_qk_pair_acc(floatx4_t &s0, floatx4_t &s1, const intx8_t &k0,
                                               const intx8_t &k1, const intx8_t &q)
{
    asm volatile("s_nop 1\n\t"
                 "v_mfma_f32_16x16x128_f8f6f4 %0, %2, %4, %0\n\t"
                 "v_mfma_f32_16x16x128_f8f6f4 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(k0), "v"(k1), "v"(q));
}

__device__ __forceinline__ void w4_qk_pad(floatx4_t &s0, floatx4_t &s1)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(s0), "+v"(s1));
}

// after_k(a) is called for a = 0, 1 once every K read of the step has
// returned (the K slots may then be refilled), in the places of row tile 0,
// which have no softmax work beside them.
template <int RT, typename AfterK>
__device__ __forceinline__ void w4_qk_softmax(RowState<RT> &st, bool &retry, bf16x8_t (&pop)[RT],
                                              floatx4_t (&S)[2][RT], const unsigned char *ka,
                                              const unsigned char *kb, const intx8_t (&qop)[RT][2][2],
                                              int ctx, int lk, int log2g, uint32_t wlim, int key0,
                                              const float (&c)[RT], int lane, AfterK after_k)
{
    const int n = lane & 15, j = lane >> 4;
    intx8_t kop[2][2];                                    // [kc][page]
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const unsigned char *kp = a ? kb : ka;
            const int c0 = 8 * kc + 2 * j;
            const uint4 lo4 = *reinterpret_cast<const uint4 *>(kp + 256 * n + 16 * (c0 ^ n));
            const uint4 hi4 = *reinterpret_cast<const uint4 *>(kp + 256 * n + 16 * ((c0 + 1) ^ n));
            kop[kc][a] = intx8_t{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                                 (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
        }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float lold[RT], mref[RT], pk[RT][2];
    uint32_t w[RT][4];
    bool need = false;
    // softmax of row tile rt, in four parts of similar issue time
    auto sm_part = [&](int rt, int part) {
        const floatx4_t &s0 = S[0][rt];
        const floatx4_t &s1 = S[1][rt];
        auto p_of = [&](float x) { return exp2_fast(__builtin_fmaf(x, c[rt], -mref[rt])); };
        // each part ends in an empty statement that takes its results, which keeps
        // the part's instructions between the MFMAs it was written between
        if (part == 0) {
            lold[rt] = st.l[rt];
            mref[rt] = st.m[rt] == -INFINITY ? 0.0f : st.m[rt];
            const float lmax = max3f(max3f(s0[0], s0[1], s0[2]), max3f(s0[3], s1[0], s1[1]), max2f(s1[2], s1[3]));
            need |= lmax * c[rt] > st.m[rt] + kTauW4;
            asm volatile("" : "+v"(mref[rt]));
        } else if (part == 1) {
            const float p0 = p_of(s0[0]), p1 = p_of(s0[1]);
            pk[rt][0] = p_of(s0[2]);
            w[rt][0] = pack_bf16x2(p0, p1);
            st.l[rt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[rt][0]), ones, st.l[rt], false);
            asm volatile("" : "+v"(w[rt][0]), "+v"(st.l[rt]), "+v"(pk[rt][0]));
        } else if (part == 2) {
            const float p3 = p_of(s0[3]);
            pk[rt][1] = p_of(s1[0]);
            const float p5 = p_of(s1[1]);
            w[rt][1] = pack_bf16x2(pk[rt][0], p3);
            st.l[rt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[rt][1]), ones, st.l[rt], false);
            pk[rt][0] = p5;
            asm volatile("" : "+v"(w[rt][1]), "+v"(st.l[rt]), "+v"(pk[rt][0]), "+v"(pk[rt][1]));
        } else {
            const float p6 = p_of(s1[2]), p7 = p_of(s1[3]);
            w[rt][2] = pack_bf16x2(pk[rt][1], pk[rt][0]);
            w[rt][3] = pack_bf16x2(p6, p7);
            st.l[rt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[rt][2]), ones, st.l[rt], false);
            st.l[rt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[rt][3]), ones, st.l[rt], false);
            asm volatile("" : "+v"(w[rt][2]), "+v"(w[rt][3]), "+v"(st.l[rt]));
            pop[rt] = __builtin_bit_cast(bf16x8_t, make_uint4(w[rt][0], w[rt][1], w[rt][2], w[rt][3]));
        }
    };
#pragma unroll
    for (int rt = 0; rt <= RT; ++rt) {
#pragma unroll
        for (int part = 0; part < 4; ++part) {
            if (rt < RT) {
                const int kc = part >> 1, h = part & 1;
                if (part == 0)
                    w4_qk_pair_first(S[0][rt], S[1][rt], kop[0][0], kop[0][1], qop[rt][0][0]);
                else
                    w4_qk_pair_acc(S[0][rt], S[1][rt], kop[kc][0], kop[kc][1], qop[rt][kc][h]);
            }
            if (rt > 0 && part == 0)
                w4_qk_pad(S[0][rt - 1], S[1][rt - 1]);
            __builtin_amdgcn_sched_barrier(0);
            if (rt > 0) {
                sm_part(rt - 1, part);
            } else if (part < 2) {
                if (part == 0)
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                after_k(part);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (__any(need)) {                                    // rare: redo the step, moving m
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            st.l[rt] = lold[rt];
        w4_softmax<RT, false, false>(st, retry, pop, S, ctx, lk, log2g, wlim, key0, true, c, 0.f, lane);
    }
}

// PV of a step: O^T += V^T P^T, as pv_lds, with the V pages of the step in two
// slots (va, vb) whose rows are stored unswizzled (chunk c of key row n at
// 256 n + 16 c): lane (m, j) reads dims 16 m .. + 15 of key rows 4 j + e, all
// of the step's V in eight 16-byte reads at one lane base plus immediates.
// after_v() is called once they have returned (the V slots may then be
// refilled).
template <int RT, typename AfterV>
__device__ __forceinline__ void w4_pv(RowState<RT> &st, const unsigned char *va, const unsigned char *vb,
                                      const bf16x8_t (&pop)[RT], bool masked, uint32_t zmask, int lane,
                                      AfterV after_v)
{
    const int m = lane & 15, j = lane >> 4;
    const int lo = 1024 * j + 16 * m;
    uint4 vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vv[e] = *reinterpret_cast<const uint4 *>((e >> 2 ? vb : va) + lo + 256 * (e & 3));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    after_v();
    if (masked) {                                      // wave-uniform
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (zmask & (1u << e))
                vv[e] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * h + qq;                  // dims 16 m + 4 q .. + 3
            uint32_t A[4][4];
#pragma unroll
            for (int kp = 0; kp < 4; ++kp) {
                const uint4 &x4 = vv[2 * kp], &y4 = vv[2 * kp + 1];
                const uint32_t X = h ? (qq ? x4.w : x4.z) : (qq ? x4.y : x4.x);
                const uint32_t Y = h ? (qq ? y4.w : y4.z) : (qq ? y4.y : y4.x);
                const uint32_t lo2 = byte_perm(Y, X, 0x05010400u);   // X0 Y0 X1 Y1
                const uint32_t hi2 = byte_perm(Y, X, 0x07030602u);   // X2 Y2 X3 Y3
                A[0][kp] = fp8x2_lo_to_bf16x2(lo2);
                A[1][kp] = fp8x2_hi_to_bf16x2(lo2);
                A[2][kp] = fp8x2_lo_to_bf16x2(hi2);
                A[3][kp] = fp8x2_hi_to_bf16x2(hi2);
            }
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) {
                const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(A[xx][0], A[xx][1], A[xx][2], A[xx][3]));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    st.o[4 * q + xx][rt] = mfma16(vop, pop[rt], st.o[4 * q + xx][rt]);
            }
        }
    }
}

// Row tile of 16 packed rows staged in LDS as bf16 (row n at 512 n, its
// 16-byte chunk c at slot c ^ n; rows n >= nr are not live and read as zero),
// converted in place into the fp8 hi / lo operands [kc][part][half][lane] x
// 16 B (the split of convert_q_block), and the rows' logit multipliers
// |c| 2^-k_n into cst[n] (Q negated when c < 0).
__device__ __forceinline__ void w4_convert_q(unsigned char *qst, float *cst, float c, int nr, int lane)
{
    const int n = lane & 15, j = lane >> 4;
    const bool live = n < nr;
    // a negative logit multiplier c is moved into the sign of Q, so that the
    // multiplier the softmax sees is >= 0
    const uint32_t flip = c < 0.f ? 0x80008000u : 0u;
    c = fabsf(c);
    uint32_t raw[2][16];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int chunk = 16 * kc + 4 * j + i;          // dims 8 chunk .. +8
            const uint4 q4 = live ? *reinterpret_cast<const uint4 *>(qst + n * 512 + ((chunk ^ n) * 16))
                                  : make_uint4(0, 0, 0, 0);
            raw[kc][4 * i] = q4.x ^ flip;
            raw[kc][4 * i + 1] = q4.y ^ flip;
            raw[kc][4 * i + 2] = q4.z ^ flip;
            raw[kc][4 * i + 3] = q4.w ^ flip;
        }
    float amax = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[kc][i] << 16)),
                                     fabsf(__builtin_bit_cast(float, raw[kc][i] & 0xFFFF0000u))));
    amax = row4_max(amax);                               // row max (4 lanes)
    int k = 0;
    if (amax > 0.f) {
        int e;
        frexpf(amax, &e);                                  // amax in [2^(e-1), 2^e)
        k = min(8 - e, 127);
    }
    if (j == 0)
        cst[n] = ldexpf(c, -k);
    // every lane has read its rows (the writes below depend on those reads)
    convert_q_block<1>(qst, raw[0], k, 0, lane);
    convert_q_block<1>(qst, raw[1], k, 1, lane);
}

// Epilogue of a w4 piece.  The four key groups hold states (m_k, l_k, O_k) of
// the same rows over disjoint keys; the piece's result is
//   O = sum_k O_k 2^(m_k - M) / W,  W = sum_k l_k 2^(m_k - M),  M = max_k m_k,
// and its log2-domain LSE is M + log2 W.  Three phases:
//   1. each wave publishes its rows' m_k, l_k (at kW4Ml of its region);
//   2. after a barrier each wave reads the four states of its rows, scales its
//      own O_k by f_k = 2^(m_k - M) / W and publishes it in fp16 (the first
//      32 KiB of its region: row r at 512 r, 16-byte chunk c at c ^ (r & 15); every
//      scaled term is a part of a convex combination of V rows, so it is at
//      most max |V| <= 448 for an e4m3 cache); wave 0 also publishes M, W;
//   3. after a barrier every thread sums the four fp16 terms of (row, 8-dim
//      chunk) items with packed fp16 adds, and writes the bf16 output row
//      (whole piece: times v_descale, with a sink in the denominator) or the
//      fp16 partial and the LSE (split piece).
typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t h2add(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v_t, a) + __builtin_bit_cast(half2v_t, b));
}

template <int RT>
__device__ __forceinline__ void w4_epilogue(RowState<RT> &st, unsigned char *lds, const SplitParams &p, int kg,
                                            int lane, int lq, int q0, int g, int slot, bool whole, float vd,
                                            bool stamp)
{
    (void)stamp;
    constexpr int NG = 4;
    const int G = 1 << p.log2g;
    // lane-derived values are formed here, from the lane index read again
    // (opaque): formed at the piece start they would be held (or spilled)
    // across the page loop
    lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane));
    const int n = lane & 15, j = lane >> 4;
    const int R = min(lq * G, 16 * RT);
    unsigned char *own = lds + kg * kW4RingBytes;
    float *ml = reinterpret_cast<float *>(own + kW4Ml);                          // [row] (m, l)
    float *mw = reinterpret_cast<float *>(lds + kW4Mw);                          // [row] (M, W), wave 0
    // the row sums of every row tile first, then their stores (between LDS
    // stores the swizzles and permutes would run one row tile at a time)
    const int x32 = (lane ^ 32) << 2;                   // the row sums' permute address, once
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        st.l[rt] += xor16_lane(st.l[rt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        st.l[rt] += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, st.l[rt])));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (16 * rt < R && j == 0) {
            ml[(16 * rt + n) * 2] = st.m[rt];
            ml[(16 * rt + n) * 2 + 1] = st.l[rt];
        }
    }
    __syncthreads();                                     // every key group's row states are out
#ifdef VA_STAMPS
    if (stamp)
        VA_STAMP(p, blockIdx.x, kg, lane, 13, VA_NOW());
#endif
    // every row tile's four states are read before any O is written: the
    // compiler cannot tell the O writes from the state reads apart, and would
    // otherwise wait out one LDS round trip per row tile (tiles past R read
    // rows nobody wrote; their factors are not used)
    float fr[RT], Mr[RT], Wr[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int row = 16 * rt + n;
        float mk[NG], lk[NG];
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const float *mlk = reinterpret_cast<const float *>(lds + k * kW4RingBytes + kW4Ml);
            mk[k] = mlk[row * 2];
            lk[k] = mlk[row * 2 + 1];
            M = fmaxf(M, lk[k] > 0.f ? mk[k] : -INFINITY);
        }
        float W = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k)
            W += lk[k] > 0.f ? lk[k] * exp2_fast(mk[k] - M) : 0.f;
        fr[rt] = (st.l[rt] > 0.f && W > 0.f) ? exp2_fast(st.m[rt] - M) / W : 0.f;
        Mr[rt] = M;
        Wr[rt] = W;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (16 * rt >= R)
            break;                                       // uniform
        const int row = 16 * rt + n;
        const float f = fr[rt];
        if (kg == 0 && j == 0) {
            mw[row * 2] = Mr[rt];
            mw[row * 2 + 1] = Wr[rt];
        }
        unsigned char *orow = own + (size_t)row * 512;
#pragma unroll
        for (int e = 0; e < 4; ++e) {                    // dims 64 j + 16 e + t, t = 0..15
            uint4 a, b;
            a.x = pack_f16x2(st.o[0][rt][e] * f, st.o[1][rt][e] * f);
            a.y = pack_f16x2(st.o[2][rt][e] * f, st.o[3][rt][e] * f);
            a.z = pack_f16x2(st.o[4][rt][e] * f, st.o[5][rt][e] * f);
            a.w = pack_f16x2(st.o[6][rt][e] * f, st.o[7][rt][e] * f);
            b.x = pack_f16x2(st.o[8][rt][e] * f, st.o[9][rt][e] * f);
            b.y = pack_f16x2(st.o[10][rt][e] * f, st.o[11][rt][e] * f);
            b.z = pack_f16x2(st.o[12][rt][e] * f, st.o[13][rt][e] * f);
            b.w = pack_f16x2(st.o[14][rt][e] * f, st.o[15][rt][e] * f);
            const int c0 = 8 * j + 2 * e;
            *reinterpret_cast<uint4 *>(orow + ((c0 ^ n) * 16)) = a;
            *reinterpret_cast<uint4 *>(orow + (((c0 + 1) ^ n) * 16)) = b;
        }
    }
#ifdef VA_STAMPS
    if (stamp)
        VA_STAMP(p, blockIdx.x, kg, lane, 14, VA_NOW());
#endif
    __syncthreads();                                     // every scaled O_k is out
#ifdef VA_STAMPS
    if (stamp)
        VA_STAMP(p, blockIdx.x, kg, lane, 15, VA_NOW());
#endif
    const int tid = kg * 64 + lane;
    const int c = tid & 31;
    // thread: chunk c of rows tid / 32 + 8 it; every row's four terms are read
    // first (rows past R re-read row R - 1 and are not stored)
    uint4 s[2 * RT];
#pragma unroll
    for (int it = 0; it < 2 * RT; ++it) {
        const int r = min((tid >> 5) + 8 * it, R - 1);
        const int off = r * 512 + ((c ^ (r & 15)) * 16);
        s[it] = *reinterpret_cast<const uint4 *>(lds + off);
#pragma unroll
        for (int k = 1; k < NG; ++k) {
            const uint4 v = *reinterpret_cast<const uint4 *>(lds + k * kW4RingBytes + off);
            s[it].x = h2add(s[it].x, v.x);
            s[it].y = h2add(s[it].y, v.y);
            s[it].z = h2add(s[it].z, v.z);
            s[it].w = h2add(s[it].w, v.w);
        }
    }
    // The stores.  Everything an item's address and scale need is copied into
    // vector registers once (free here): kept in scalar registers, the kernel's
    // parameters are restored from their spill lanes for every item.
    const int r0 = tid >> 5;
    if (whole) {
        uint64_t ob = reinterpret_cast<uint64_t>(p.out + 8 * c);
        int rowb = q0 * p.hq + g * G, hq = p.hq, lg = p.log2g;
        float vdv = vd;
        uint64_t sk = reinterpret_cast<uint64_t>(p.sinks ? p.sinks + g * G : nullptr);
        asm volatile("" : "+v"(ob), "+v"(rowb), "+v"(hq), "+v"(lg), "+v"(vdv), "+v"(sk));
        const bool has_sinks = p.sinks != nullptr;
#pragma unroll
        for (int it = 0; it < 2 * RT; ++it) {
            const int r = r0 + 8 * it;
            if (r >= R)
                break;
            const float M = mw[r * 2], W = mw[r * 2 + 1];
            const int t = r >> lg, h = r & ((1 << lg) - 1);
            float sc = W > 0.f ? vdv : 0.f;
            if (has_sinks) {                             // the sink joins the denominator only
                const float skl = reinterpret_cast<const float *>(sk)[h] * 1.4426950408889634f;
                const float mm = fmaxf(M, skl);
                const float Wf = W > 0.f ? W * exp2_fast(M - mm) : 0.f;
                sc = vdv * Wf / (Wf + exp2_fast(skl - mm));
            }
            uint4 o;
            o.x = pack_bf16x2(f16_lo(s[it].x) * sc, f16_hi(s[it].x) * sc);
            o.y = pack_bf16x2(f16_lo(s[it].y) * sc, f16_hi(s[it].y) * sc);
            o.z = pack_bf16x2(f16_lo(s[it].z) * sc, f16_hi(s[it].z) * sc);
            o.w = pack_bf16x2(f16_lo(s[it].w) * sc, f16_hi(s[it].w) * sc);
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(ob) +
                                       (int64_t)(rowb + t * hq + h) * kHeadDim) = o;
        }
    } else {                                             // fp16 partial O / l as summed, and the LSE
        const int64_t row0 = (int64_t)slot * p.rows_max;
        uint64_t wb = reinterpret_cast<uint64_t>(static_cast<uint16_t *>(p.ws_o) + row0 * kHeadDim + 8 * c);
        uint64_t lb = reinterpret_cast<uint64_t>(p.ws_lse + row0);
        asm volatile("" : "+v"(wb), "+v"(lb));
#pragma unroll
        for (int it = 0; it < 2 * RT; ++it) {
            const int r = r0 + 8 * it;
            if (r >= R)
                break;
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(wb) + (int64_t)r * kHeadDim) = s[it];
            if (c == 0) {
                const float M = mw[r * 2], W = mw[r * 2 + 1];
                reinterpret_cast<float *>(lb)[r] = W > 0.f ? M + __log2f(W) : -INFINITY;
            }
        }
    }
}

template <int RT, bool CAP>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void va_split_kv_fp8_w4_kernel(SplitParams p)
{
    constexpr int NG = 4;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NG * kW4RingBytes];

    const int lane = threadIdx.x & 63;
    const int kg = uniform(threadIdx.x >> 6);
    const int w = blockIdx.x;
    const int G = 1 << p.log2g;
    VA_STAMP(p, w, kg, lane, 0, VA_NOW());

    Share sh = locate(p, w, lane, w == 0 && kg == 0);
    sh.n_eff = uniform(sh.n_eff);
    sh.s = uniform(sh.s);
    sh.e = uniform(sh.e);
    sh.bg = uniform(sh.bg);
    sh.base = uniform(sh.base);
    sh.q0 = uniform(sh.q0);
    sh.q1 = uniform(sh.q1);
    sh.lk = uniform(sh.lk);
    if (w >= sh.n_eff)
        return;                                        // uniform over the workgroup
    VA_STAMP(p, w, kg, lane, 1, VA_NOW());
#ifdef VA_STAMPS
    int npieces = 0;
    VA_STAMP(p, w, kg, lane, 11, (unsigned long long)__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)));
#endif

    const float kd = load_descale(p.kdesc);
    const float vd = load_descale(p.vdesc);
    unsigned char *ring = lds + kg * kW4RingBytes;
    const uint32_t ring_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(ring));
    const int64_t page_bytes = (int64_t)kPage * p.hkv * kHeadDim;

    const int bh = p.num_seqs * p.hkv;
    int s = sh.s, bg = sh.bg, base = sh.base;
    while (s < sh.e && bg < bh) {
        int pl = lane;                                 // opaque per piece (see the w8 kernel)
        asm volatile("" : "+v"(pl));
        uint32_t off[4];
        dma_lane_offsets(off, p.hkv, pl);
        const int b = uniform(bg / p.hkv);
        const int g = bg - b * p.hkv;
        int hdr[3];                                            // cu[b], cu[b + 1], seqused[b]
        if (bg == sh.bg) {                                     // loaded by locate() already
            hdr[0] = sh.q0;
            hdr[1] = sh.q1;
            hdr[2] = sh.lk;
        } else {
            load_uniform3(hdr, p.cu + b, p.cu + b + 1, p.seqused + b);
        }
        const int q0 = hdr[0];
        const int lq = checked_q_len(q0, hdr[1], p.total_q, p.max_q);
        const int lk = hdr[2];
        const int pb = first_page(lk, lq, p.window_left);      // the range starts at logical page pb
        const int cnt = (lq <= 0 || lk <= 0) ? 0 : max(0, min((lk + kPage - 1) / kPage, p.mbps) - pb);
        if (cnt == 0) {
            ++bg;
            continue;
        }
        const int ctx = lk - lq;
        const int r0 = s - base;                               // piece = pages r0 .. r1 of the pair's range
        const int r1 = min(sh.e, base + cnt) - base;
        const bool whole = (r0 == 0 && r1 == cnt);
        const int p0 = pb + r0, p1 = pb + r1;
        const int slot = 2 * w + (s != sh.s);           // first or last piece of this workgroup
        const int lo_max = p.window_left < 0 ? INT_MIN : ctx + lq - 1 - p.window_left;
        const uint32_t wlim = p.window_left < 0 ? 0x7FFFFFFFu : (uint32_t)p.window_left;

        // Wave kg computes a contiguous quarter of the piece's page pairs, so the
        // block-table entries of its pages are consecutive.  Its local page i is
        // logical page lp0 + i; the missing second page of the piece's last pair
        // (an odd page count) re-reads the first, and its keys are masked.
        const int npairs = (p1 - p0 + 1) >> 1;
        const int pr0 = (int)(((int64_t)kg * npairs) / NG);
        const int nst = (int)(((int64_t)(kg + 1) * npairs) / NG) - pr0;   // steps of this wave
        const int lp0 = p0 + 2 * pr0;
        const int32_t *btrow = p.bt + (int64_t)b * p.mbps;
        const uint8_t *kpool = p.k + (int64_t)g * kHeadDim;
        const uint8_t *vpool = p.v + (int64_t)g * kHeadDim;
        const int maxpage = (int)min(p.num_blocks - 1, (int64_t)INT_MAX);
        auto entry = [&](int i) -> int {                       // pool page of local page i, clamped
            const int pg = min(lp0 + i, p1 - 1);
            const int y = load_uniform(btrow, pg);
            return y < 0 ? 0 : (y > maxpage ? maxpage : y);
        };
        auto issue_k = [&](int y, int slot_i) {                // K of pool page y into K slot slot_i
            const uint8_t *src_pg = kpool + (int64_t)y * page_bytes;
            const uint32_t dst = ring_addr + (uint32_t)(slot_i * kW4PageBytes);
#pragma unroll
            for (int x = 0; x < 4; ++x)
                dma16(src_pg, off[x], dst + 1024 * x);
        };
        uint32_t off_v[4];                                     // V rows are stored unswizzled
#pragma unroll
        for (int x = 0; x < 4; ++x)
            off_v[x] = (uint32_t)((4 * x + (pl >> 4)) * p.hkv * kHeadDim + 16 * (pl & 15));
        auto issue_v = [&](int y, int slot_i, int x0 = 0, int x1 = 4) {   // V of pool page y (rows 4 x0 ..
            const uint8_t *src_pg = vpool + (int64_t)y * page_bytes;     // 4 x1 - 1) into V slot slot_i
            const uint32_t dst = ring_addr + (uint32_t)(kW4VBase + slot_i * kW4PageBytes);
#pragma unroll
            for (int x = x0; x < x1; ++x)
                dma16(src_pg, off_v[x], dst + 1024 * x);
        };

        // ---- prologue
        __syncthreads();                                       // previous piece's LDS reads done
        const int R = lq * G;
        const int nr = min(max(R - 16 * kg, 0), 16);           // live rows of row tile kg
        unsigned char *qst = ring + kW4QStage;
        float *cst = reinterpret_cast<float *>(ring + kW4CStage);
        for (int i = 0; 2 * i < nr; ++i) {                     // row pairs (G is even): 1 KiB each
            const int r = 16 * kg + 2 * i;
            const int64_t row0 = uniform((int)((int64_t)(q0 + (r >> p.log2g)) * p.hq + g * G + (r & (G - 1))));
            const int rr = 2 * i + (pl >> 5), sl = pl & 31;    // lane's LDS row and slot
            dma16(p.q + row0 * kHeadDim, (uint32_t)((pl >> 5) * 512 + ((sl ^ (rr & 15)) * 16)),
                  ring_addr + (uint32_t)(kW4QStage + 2 * i * 512));
        }
        // The block-table entries of the first five steps' pages, in one batch of
        // scalar loads while the Q rows are in flight: one latency, none at step 0.
        int ent[10];
        load_entries10(ent, btrow, lp0, p1 - 1);
#pragma unroll
        for (int i = 0; i < 10; ++i)
            ent[i] = ent[i] < 0 ? 0 : (ent[i] > maxpage ? maxpage : ent[i]);
        // With the Q rows go K and V of pages 0 .. 3 (31 copies: the last KiB of
        // V page 3 is the exchange's multiplier area); after the exchange that
        // KiB and K of pages 4, 5 (the exchange's row area).  Issue order, which
        // the waits below count: K(0) V(0) K(1) V(1)' | V(1)'' K(2).
        auto prologue_copies = [&](int part) {
            if (part == 0) {
                if (nst > 0) {
                    issue_k(ent[0], 0);
                    issue_k(ent[1], 1);
                    issue_v(ent[0], 0);
                    issue_v(ent[1], 1);
                }
                if (nst > 1) {
                    issue_k(ent[2], 2);
                    issue_k(ent[3], 3);
                    issue_v(ent[2], 2);
                    issue_v(ent[3], 3, 0, 3);
                }
            } else {
                if (nst > 1)
                    issue_v(ent[3], 3, 3, 4);
                if (nst > 2) {
                    issue_k(ent[4], 4);
                    issue_k(ent[5], 5);
                }
            }
        };
        prologue_copies(0);
        RowState<RT> st;                                       // O starts at zero
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            st.m[rt] = -INFINITY;
#pragma unroll
            for (int t = 0; t < 16; ++t)
                st.o[t][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (nst > 1)
            wait_vmcnt<31>();                                  // this wave's Q copies landed
        else if (nst > 0)
            wait_vmcnt<16>();
        else
            wait_vmcnt<0>();
#ifdef VA_STAMPS
        const bool first_piece = npieces++ == 0;
        if (first_piece)
            VA_STAMP(p, w, kg, lane, 2, VA_NOW());
#endif
        if (kg < RT) {
            // the logit multiplier, formed here from scalar registers: a vector
            // copy kept across the pieces is spilled, and its reload would wait
            // for every copy in flight
            float kdp = kd;
            asm volatile("" : "+s"(kdp));
            w4_convert_q(qst, cst, p.scale_log2 * kdp, nr, pl);
        }
        __syncthreads();                                       // every row tile converted
        intx8_t qop[RT][2][2];
        float crow[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const unsigned char *qs = lds + rt * kW4RingBytes + kW4QStage + pl * 16;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    const uint4 b0 = *reinterpret_cast<const uint4 *>(qs + (kc * 2 + part) * 2048);
                    const uint4 b1 = *reinterpret_cast<const uint4 *>(qs + (kc * 2 + part) * 2048 + 1024);
                    qop[rt][kc][part] = intx8_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                                (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                }
            crow[rt] = reinterpret_cast<const float *>(lds + rt * kW4RingBytes + kW4CStage)[pl & 15];
        }
        __syncthreads();                                       // every wave holds the operands
#ifdef VA_STAMPS
        if (first_piece)
            VA_STAMP(p, w, kg, lane, 3, VA_NOW());
#endif
        prologue_copies(1);

        for (int pass = 0;; ++pass) {                          // a second pass only after `retry`
            if (pass > 0) {
                prologue_copies(0);
                prologue_copies(1);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        st.o[t][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                st.l[rt] = 0.f;
            bool retry = false;
            // Copies: the prologue issues K(0), V(0), K(1), V(1), K(2) (X(s) = the two
            // pages of step s; the last KiB of V(1) just before K(2)); step t then
            // refills its own slots as soon as it has read them: K(t + 3) once its K
            // reads have returned, V(t + 2) once its V reads have.  Block-table
            // entries at the start of step t: eK for K(t + 3) (pages 2t + 6, 2t + 7),
            // eV for V(t + 2) (pages 2t + 4, 2t + 5), eN for the next step's K (pages
            // 2t + 8, 2t + 9), loaded a step ahead (entry() clamps to the piece, so
            // the loads past its end are harmless).
            int eK0 = ent[6], eK1 = ent[7], eV0 = ent[4], eV1 = ent[5];
            int eN0 = ent[8], eN1 = ent[9];
            int ks = 0, vs = 0;                                // K / V slots of local page 2t
#ifdef VA_STAMPS
            uint32_t sl[8] = {0, 0, 0, 0, 0, 0, 0, 0};       // the loop's stamps (low 32 bits), held
#endif
            for (int t = 0; t < nst; ++t) {
#ifdef VA_STAMPS
                const bool mid = first_piece && pass == 0 && t == (nst >> 1);
#endif
                // K(t) must have landed.  Issued after it so far (in issue order, each
                // 8 copies): V(t), K(t+1) and V(t+1) if t+1 < nst, K(t+2) if t+2 < nst;
                // from t = 3 on also V(t-1) (V(1) precedes K(2))
                wait_vmcnt_x8(8 * ((t >= 3 ? 2 : 1) + 2 * (t + 1 < nst) + (t + 2 < nst)));
#ifdef VA_STAMPS
                if (first_piece && pass == 0 && t <= 1)
                    sl[t] = (uint32_t)VA_NOW();
                if (mid) {
                    sl[2] = (uint32_t)VA_NOW();
                    sl[6] = (uint32_t)__builtin_amdgcn_s_memtime();
                }
#endif
                const int kslot = ks, vslot = vs;
                const unsigned char *ka = ring + ks * kW4PageBytes;
                const unsigned char *va = ring + kW4VBase + vs * kW4PageBytes;
                ks = ks + 2 == kW4KSlots ? 0 : ks + 2;
                vs = vs + 2 == kW4VSlots ? 0 : vs + 2;
                auto after_k = [&](int a) {                    // K(t + 3) into this step's K slots
                    if (t + 3 < nst)
                        issue_k(a ? eK1 : eK0, kslot + a);
                };
                auto after_v = [&]() {                         // V(t + 2) into this step's V slots
                    if (t + 2 < nst) {
                        issue_v(eV0, vslot);
                        issue_v(eV1, vslot + 1);
                    }
                };
                // lane-derived LDS offsets are rederived each step from an
                // opaque lane index: hoisted out of the loop they would hold
                // registers next to the Q operands
                int ln = lane;
                asm volatile("" : "+v"(ln));
                floatx4_t S[2][RT];
                const int pa = lp0 + 2 * t;
                const bool hb = pa + 1 < p1;
                const int key0 = pa * kPage;
                bf16x8_t pop[RT];
                // uniform: a causal, length or window edge.  Only QK and the softmax have
                // two versions: two copies of the PV would give O two definitions per step
                const bool masked = !hb || key0 + 31 > ctx || key0 < lo_max;
                if (CAP || masked) {
                    w4_qk<RT>(S, ka, ka + kW4PageBytes, qop, ln);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    after_k(0);
                    after_k(1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (masked)
                        w4_softmax<RT, CAP, true>(st, retry, pop, S, ctx, lk, p.log2g, wlim, key0, hb, crow,
                                                  p.cap_log2, ln);
                    else
                        w4_softmax<RT, CAP, false>(st, retry, pop, S, ctx, lk, p.log2g, wlim, key0, hb, crow,
                                                   p.cap_log2, ln);
                } else {
                    w4_qk_softmax<RT>(st, retry, pop, S, ka, ka + kW4PageBytes, qop, ctx, lk, p.log2g, wlim, key0,
                                      crow, ln, after_k);
                }
#ifdef VA_STAMPS
                if (mid)
                    sl[3] = (uint32_t)VA_NOW();
#endif
                // V(t) must have landed.  Issued after it so far: V(t+1), K(t+2) and
                // K(t+3) where those steps exist, and at t = 0, 1 also K(t+1)
                wait_vmcnt_x8(8 * ((t + 1 < nst) * (t <= 1 ? 2 : 1) + (t + 2 < nst) + (t + 3 < nst)));
#ifdef VA_STAMPS
                if (mid)
                    sl[4] = (uint32_t)VA_NOW();
#endif
                __builtin_amdgcn_sched_barrier(0);
                w4_pv<RT>(st, va, va + kW4PageBytes, pop, masked, masked ? v_zero_mask(key0, hb, lk, ln) : 0u, ln,
                          after_v);
#ifdef VA_STAMPS
                if (mid) {
                    sl[5] = (uint32_t)VA_NOW();
                    sl[7] = (uint32_t)__builtin_amdgcn_s_memtime();
                }
#endif
                eV0 = eK0;
                eV1 = eK1;
                eK0 = eN0;
                eK1 = eN1;
                eN0 = entry(2 * t + 10);
                eN1 = entry(2 * t + 11);
            }
            wait_vmcnt<0>();
            if (!__any(retry) || pass == 1) {                  // a second pass cannot move m again
#ifdef VA_STAMPS
                if (first_piece) {
                    VA_STAMP(p, w, kg, lane, 6, VA_NOW());
                    VA_STAMP(p, w, kg, lane, 9, (unsigned long long)nst);
                    VA_STAMP(p, w, kg, lane, 12, (unsigned long long)(pass + 1));
                    VA_STAMP(p, w, kg, lane, 4, (unsigned long long)sl[0]);
                    VA_STAMP(p, w, kg, lane, 5, (unsigned long long)sl[1]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        VA_STAMP(p, w, kg, lane, 16 + i, (unsigned long long)sl[2 + i]);
                    VA_STAMP(p, w, kg, lane, 20, (unsigned long long)sl[6]);
                    VA_STAMP(p, w, kg, lane, 21, (unsigned long long)sl[7]);
                }
#endif
                break;
            }
        }

#ifdef VA_STAMPS
        w4_epilogue<RT>(st, lds, p, kg, pl, lq, q0, g, slot, whole, vd, first_piece);
#else
        w4_epilogue<RT>(st, lds, p, kg, pl, lq, q0, g, slot, whole, vd, false);
#endif
#ifdef VA_STAMPS
        if (first_piece)
            VA_STAMP(p, w, kg, lane, 7, VA_NOW());
#endif

        s = base + r1;
        base += cnt;
        ++bg;
    }
#ifdef VA_STAMPS
    VA_STAMP(p, w, kg, lane, 8, VA_NOW());
    VA_STAMP(p, w, kg, lane, 10, (unsigned long long)npieces);
#endif
}

// ------------------------------------------------- bf16 cache, LDS design --
//
// The same workgroup shape as the FP8 kernel (8 waves: 4 key groups x 2 row
// groups, 2-stage ring per key group, direct global->LDS copies), with one
// page (16 keys) per step: a stage holds the K page and the V page of one kv
// head, 8 KiB each (16 rows of 512 bytes; the 16-byte chunk c of key row n sits
// at slot c ^ (n & 15)).  QK runs on v_mfma_f32_16x16x32_bf16 with Q taken as
// stored (bf16 operands copied into LDS in operand order, no conversion); PV
// on v_mfma_f32_16x16x16_bf16 (K = the 16 keys of the page), its V^T operands
// transposed from the key rows with byte permutes.

typedef short shortx4_t __attribute__((ext_vector_type(4)));
constexpr int kQbf16Bytes = 4 * 8 * 64 * 16;                // [rt][s][lane] x 16 B: 4 row tiles

__device__ __forceinline__ floatx4_t mfma16k16(const shortx4_t &a, const shortx4_t &b, const floatx4_t &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Lane offsets of the 8 copy instructions of one bf16 page: instruction i,
// lane l writes LDS bytes [1024 i + 16 l, +16) = key row n = 2 i + l/32, slot
// l%32, so it fetches chunk (l%32) ^ (n & 15) of that key row.
__device__ __forceinline__ void dma_lane_offsets_bf16(uint32_t (&off)[8], int hkv, int lane)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int n = 2 * i + (lane >> 5);
        off[i] = (uint32_t)(n * hkv * kHeadDim * 2 + (((lane & 31) ^ (n & 15)) * 16));
    }
}

__device__ __forceinline__ void dma_page_bf16(uint32_t dst, const uint8_t *pool, int64_t y, int64_t page_bytes,
                                              const uint32_t (&off)[8])
{
    const uint8_t *a = pool + y * page_bytes;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dma16(a, off[i], dst + 1024 * i);
}

// S^T[rt] (16 keys x 16 rows) of one page: K operand of lane (n = l%16, j =
// l/16) for dims 32 s + 8 j .. +8 of key n = chunk 4 s + j.
template <int RTW>
__device__ __forceinline__ void qk_lds_bf16(floatx4_t (&S)[RTW], const unsigned char *stage,
                                            const unsigned char *qw, int lane)
{
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
        S[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t *>(stage + 512 * n + (((4 * s + j) ^ n) * 16));
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const bf16x8_t qop = *reinterpret_cast<const bf16x8_t *>(qw + ((size_t)(rt * 8 + s) * 64 + lane) * 16);
            S[rt] = mfma16(kop, qop, S[rt]);
        }
    }
}

// Online softmax of a one-page step: lane (row n, j) holds the logits of keys
// key0 + 4 j + e, e = 0..3; returns P^T B-operands (4 bf16).  Same rules as
// softmax_step.
template <int RTW, bool CAP>
__device__ __forceinline__ void softmax_step1(RowState<RTW> &st, shortx4_t (&pop)[RTW], const floatx4_t (&S)[RTW],
                                              const int (&limit)[RTW], uint32_t wlim, int key0, float c,
                                              float cap, int lane, bool masked)
{
    const int j = lane >> 4;
    float x[RTW][4];
    bool need_any = false;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = S[rt][e] * c;
            if constexpr (CAP)
                v = softcap_log2(v, cap);
            if (masked) {
                const int key = key0 + 4 * j + e;
                v = (uint32_t)(limit[rt] - key) <= wlim ? v : -INFINITY;
            }
            x[rt][e] = v;
        }
        const float lmax = fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3]));
        need_any |= lmax > st.m[rt] + kTau;
    }
    if (__any(need_any)) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            float t = fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3]));
            t = fmaxf(t, __shfl_xor(t, 16));
            t = fmaxf(t, __shfl_xor(t, 32));
            const bool need = t > st.m[rt] + kTau;
            const float alpha = need ? exp2_fast(st.m[rt] - t) : 1.0f;
            st.m[rt] = need ? t : st.m[rt];
            st.l[rt] *= alpha;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt)
                st.o[tt][rt] *= alpha;
        }
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const float mref = st.m[rt] == -INFINITY ? 0.0f : st.m[rt];
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pv[e] = exp2_fast(x[rt][e] - mref);
        st.l[rt] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        pop[rt] = __builtin_bit_cast(shortx4_t, make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])));
    }
}

// PV of a one-page step: lane (m = l%16, j = l/16) reads dims 16 m .. 16 m + 15
// of keys 4 j + e (two 16-byte chunks per key row) and builds, for dim tile T,
// the V^T operand {V[4j + e][16 m + T], e = 0..3}.  zmask bit e zeroes key
// 4 j + e (at or past seqused_k: it may hold NaN bytes).
template <int RTW>
__device__ __forceinline__ void pv_lds_bf16(RowState<RTW> &st, const unsigned char *stage,
                                            const shortx4_t (&pop)[RTW], uint32_t zmask, int lane)
{
    const int m = lane & 15, j = lane >> 4;
    const unsigned char *vb = stage + 8192;
    uint4 v[4][2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int n = 4 * j + e;
        v[e][0] = *reinterpret_cast<const uint4 *>(vb + 512 * n + (((2 * m) ^ n) * 16));
        v[e][1] = *reinterpret_cast<const uint4 *>(vb + 512 * n + (((2 * m + 1) ^ n) * 16));
    }
    if (zmask) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (zmask & (1u << e)) {
                v[e][0] = make_uint4(0, 0, 0, 0);
                v[e][1] = make_uint4(0, 0, 0, 0);
            }
    }
#pragma unroll
    for (int T = 0; T < 16; ++T) {
        const int h = T >> 3, d = (T & 7) >> 1;
        const uint32_t sel = (T & 1) ? 0x07060302u : 0x05040100u;     // high or low bf16 of each dword
        const uint32_t w0 = byte_perm(u4get(v[1][h], d), u4get(v[0][h], d), sel);
        const uint32_t w1 = byte_perm(u4get(v[3][h], d), u4get(v[2][h], d), sel);
        const shortx4_t a = __builtin_bit_cast(shortx4_t, make_uint2(w0, w1));
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
            st.o[T][rt] = mfma16k16(a, pop[rt], st.o[T][rt]);
    }
}

// bf16 split-KV kernel, LDS design.  Same structure as the FP8 kernel: the two
// waves of a key group share a 2-stage ring (one copies each step's K page,
// the other its V page), the prologue copies the Q operands and the first two
// steps, one barrier per step.
template <int RTW, bool CAP, bool TOK>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void va_split_kv_bf16_w8_kernel(SplitParams p)
{
    constexpr int NG = 4;
    constexpr int RT = 2 * RTW;
    constexpr int kQBytes = kQbf16Bytes;
    constexpr int kRingBytes = 2 * kStageBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kQBytes + NG * kRingBytes];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int rg = wave & 1;
    const int kg = wave >> 1;
    const int w = blockIdx.x;
    const int G = 1 << p.log2g;

    Share sh = locate(p, w, lane, w == 0 && wave == 0);
    sh.n_eff = uniform(sh.n_eff);
    sh.s = uniform(sh.s);
    sh.e = uniform(sh.e);
    sh.bg = uniform(sh.bg);
    sh.base = uniform(sh.base);
    if (w >= sh.n_eff)
        return;                                        // uniform over the workgroup

    const float kd = load_descale(p.kdesc);
    const float vd = load_descale(p.vdesc);
    const float c = p.scale_log2 * kd;
    unsigned char *ring = lds + kQBytes + kg * kRingBytes;
    const uint32_t ring_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(ring));
    const uint32_t lds_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(lds));
    const unsigned char *qw = lds + (size_t)rg * RTW * 8 * 64 * 16;
    const int64_t page_bytes = (int64_t)kPage * p.hkv * kHeadDim * 2;

    const int bh = p.num_seqs * p.hkv;
    int s = sh.s, bg = sh.bg, base = sh.base;
    while (s < sh.e && bg < bh) {
        int pl = lane;                                 // opaque per piece (see the FP8 kernel)
        asm volatile("" : "+v"(pl));
        uint32_t off[8];
        dma_lane_offsets_bf16(off, p.hkv, pl);
        const int b = uniform(bg / p.hkv);
        const int g = bg - b * p.hkv;
        const int q0 = load_uniform(p.cu, b);
        const int lq = checked_q_len(q0, load_uniform(p.cu, b + 1), p.total_q, p.max_q);
        int s0 = 0, lk;                                        // s0: prefix start in kv_indices
        if constexpr (TOK) {
            s0 = load_uniform(p.kv_indptr, b);
            lk = prefix_keys(s0, load_uniform(p.kv_indptr, b + 1), lq, p.num_indices);
        } else {
            lk = load_uniform(p.seqused, b);
        }
        const int pb = first_page(lk, lq, p.window_left);
        const int cnt = (lq <= 0 || lk <= 0) ? 0 : max(0, min((lk + kPage - 1) / kPage, p.mbps) - pb);
        if (cnt == 0) {
            ++bg;
            continue;
        }
        const int ctx = lk - lq;
        const int r0 = s - base;
        const int r1 = min(sh.e, base + cnt) - base;
        const bool whole = (r0 == 0 && r1 == cnt);
        const int p0 = pb + r0;
        const int slot = 2 * w + (s != sh.s);           // first or last piece of this workgroup
        const int lo_max = p.window_left < 0 ? INT_MIN : ctx + lq - 1 - p.window_left;
        const uint32_t wlim = p.window_left < 0 ? 0x7FFFFFFFu : (uint32_t)p.window_left;

        const int nst = r1 - r0;                               // pages = steps of the piece
        const int nsteps = (nst + NG - 1) / NG;                // uniform over the workgroup
        const bool rows_live = (rg * RTW * 16) < lq * G;
        const int32_t *btrow = p.bt + (int64_t)b * p.mbps;
        const uint8_t *pool = (rg == 0 ? p.k : p.v) + (int64_t)g * kHeadDim * 2;
        const int64_t maxpage = p.num_blocks - 1;
        auto issue = [&](int k, int stage) {                   // this wave's page of step k
            int64_t y = load_uniform(btrow, uniform(p0 + k));
            y = y < 0 ? 0 : (y > maxpage ? maxpage : y);
            dma_page_bf16(ring_addr + stage * kStageBytes + 8192 * rg, pool, y, page_bytes, off);
        };
        // prefix + extend layout (see the FP8 kernel): lane l tags key
        // 16 (p0 + k) + l % 16; copy i takes key row n = 2 i + l / 32.
        const int pre = lk - lq;
        const uint8_t *ext = (rg == 0 ? p.kext : p.vext) + (int64_t)g * kHeadDim * 2;
        const int64_t row_bytes = (int64_t)p.hkv * kHeadDim * 2;
        auto tload = [&](int k) { return tok_load(p, b, s0, pre, (p0 + k) * kPage + (pl & 15)); };
        auto issue_tok = [&](int k, int stage, int32_t raw) {
            const int32_t tag = tok_tag(raw, (p0 + k) * kPage + (pl & 15), pre, lk, q0, p.num_rows);
            const uint32_t dst = ring_addr + stage * kStageBytes + 8192 * rg;
            int32_t t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t[i] = __shfl(tag, 2 * i + (pl >> 5));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int n = 2 * i + (pl >> 5);
                dma16_at(tok_row(t[i], pool, ext, row_bytes) + (((pl & 31) ^ (n & 15)) * 16), dst + 1024 * i);
            }
        };
        int32_t rawA = 0, rawB = 0, rawN = 0;
        if constexpr (TOK) {
            rawA = tload(kg);
            rawB = tload(kg + NG);
            asm volatile("" : "+v"(rawA), "+v"(rawB));
        }

        // ---- prologue: Q operands and the first two steps' pages
        __syncthreads();                                       // previous piece's LDS reads done
        {
            // instruction i = rt * 8 + s: lane l gets dims 32 s + 8 (l/16) .. +8 of
            // packed row 16 rt + l%16 (rows past the piece's tokens re-read token 0)
            const uint16_t *qbase = p.q + ((int64_t)q0 * p.hq + g * G) * kHeadDim;
            for (int i = wave; i < RT * 8; i += 2 * NG) {
                const int rt = i >> 3, sc = i & 7;
                const int r = 16 * rt + (pl & 15);
                int t = r >> p.log2g;
                t = t < lq ? t : 0;
                const uint32_t voff = (uint32_t)(((t * p.hq + (r & (G - 1))) * kHeadDim + 32 * sc + 8 * (pl >> 4)) * 2);
                dma16(qbase, voff, lds_addr + i * 1024);
            }
        }
        const bool has1 = kg + NG < nst;
        if (kg < nst) {
            if constexpr (TOK)
                issue_tok(kg, 0, rawA);
            else
                issue(kg, 0);
        }
        if (has1) {
            if constexpr (TOK) {
                issue_tok(kg + NG, 1, rawB);
                rawN = tload(kg + 2 * NG);
            } else {
                issue(kg + NG, 1);
            }
        }
        if (has1)
            wait_vmcnt<TOK ? 17 : 16>();                       // this wave's Q copies landed
        else if (kg < nst)
            wait_vmcnt<8>();
        else
            wait_vmcnt<0>();

        RowState<RTW> st;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            st.m[rt] = -INFINITY;
            st.l[rt] = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t)
                st.o[t][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
        int limit[RTW];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const int t = ((rg * RTW + rt) * 16 + (pl & 15)) >> p.log2g;
            limit[rt] = min(ctx + t, lk - 1);
        }

        for (int t = 0; t < nsteps; ++t) {
            const int k = kg + t * NG;
            if (t == 0 && k + NG < nst)
                wait_vmcnt<TOK ? 9 : 8>();                     // own copies of step 0 landed
            else
                wait_vmcnt<0>();
            if constexpr (TOK) {
                if (t >= 1)
                    asm volatile("" : "+v"(rawN));
            }
            __syncthreads();                                   // partner's too (and all Q copies)
            if (t >= 1 && k + NG < nst) {
                if constexpr (TOK) {
                    issue_tok(k + NG, (t + 1) & 1, rawN);
                    rawN = tload(k + 2 * NG);
                } else {
                    issue(k + NG, (t + 1) & 1);
                }
            }
            if (k < nst && rows_live) {
                const unsigned char *stage = ring + (t & 1) * kStageBytes;
                floatx4_t S[RTW];
                qk_lds_bf16<RTW>(S, stage, qw, pl);
                const int key0 = (p0 + k) * kPage;
                const bool masked = key0 + 15 > ctx || key0 < lo_max;
                shortx4_t pop[RTW];
                softmax_step1<RTW, CAP>(st, pop, S, limit, wlim, key0, c, p.cap_log2, pl, masked);
                uint32_t zmask = 0;
                if (masked) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (key0 + 4 * (pl >> 4) + e >= lk)
                            zmask |= 1u << e;
                }
                pv_lds_bf16<RTW>(st, stage, pop, zmask, pl);
            }
        }
        wait_vmcnt<0>();

        piece_epilogue<RTW, kKvBf16>(st, lds, lds + kQBytes, p, kg, rg, pl, lq, q0, g, slot, whole, vd);

        s = base + r1;
        base += cnt;
        ++bg;
    }
}

// ------------------------------------------------ absorbed MLA (PE_DIM split) --
//
// One kv head whose cache row is [latent (512) | RoPE part (64)]: 576 values,
// 576 bytes (FP8) or 1152 bytes (bf16) per key.  The logit of a query row
// [q_nope | q_pe] is the dot product over the whole row (q_nope.k_nope +
// q_pe.k_pe); the value of a key is its latent.  Each key row is copied into
// LDS once and serves both contractions.
//
// Workgroup: 8 waves = 2 key groups x 4 row tiles of the packed rows
// r = t G + h (up to 64).  Key group kg takes pages kg, kg + 2, ... of the
// piece; its 4 waves share a 2-stage LDS ring of one page per stage.  Each wave
// computes, for its own row tile, S^T = K Q^T over the 576 dims, its own
// online softmax and O^T += V^T P^T over the 512 latent dims (32 O^T tiles,
// 128 registers).  The two key groups merge in the epilogue.
//
// Ring rows: row n of a page sits at n * row bytes, its 16-byte chunk c at slot
// c ^ swz(n), swz = ((n >> 2) ^ (n >> 3)) & 1 | ((n >> 2) & 1) << 1 (FP8, 36
// chunks a row) or n & 7 (bf16, 72 chunks a row).  Both were chosen by
// measuring LDS bank conflicts (SQ_LDS_BANK_CONFLICT) of the kernel's read
// patterns on gfx950: QK reads one chunk of 16 rows, PV reads transposed
// (mla_pv_f8, mla_pv_bf16); none of them conflicts.  (n >> 2) & 3 costs a
// two-way conflict on the FP8 QK reads, ((n >> 2) ^ (n >> 3)) & 3 one on the
// FP8 transposed reads, (n >> 1) & 7 one on the bf16 transposed reads.  A page copy is 9 (FP8) or 18 (bf16) 1-KiB copies; wave (kg, rt)
// issues copies rt, rt + 4, ... of its key group's page.

constexpr int kMlaDim = 576;                   // cache row and query row width
constexpr int kMlaDv = 512;                    // latent = value width
constexpr int kMlaRows = 64;                   // packed rows: up to 16 heads x 4 tokens
constexpr int kMlaObufBytes = 2 * kMlaRows * kMlaDv * 2;   // epilogue: [kg][row][512] x 2 B

template <int KVT> struct MlaCfg;
template <> struct MlaCfg<kKvFp8> {
    static constexpr int kRowBytes = kMlaDim;
    static constexpr int kChunks = 36;
    static constexpr int kCopies = 9;
    static constexpr int kMaxCopies = 3;                   // wave rt = 0; the others 2
    static constexpr int kPages = 2;                       // pages per key-group step
    static constexpr int kQBytes = 4 * 5 * 2 * 64 * 32;     // [rt][c][hi, lo][half][lane] x 16 B
    __device__ static int swz(int n) { return (((n >> 2) ^ (n >> 3)) & 1) | (((n >> 2) & 1) << 1); }
};
template <> struct MlaCfg<kKvBf16> {
    static constexpr int kRowBytes = 2 * kMlaDim;
    static constexpr int kChunks = 72;
    static constexpr int kCopies = 18;
    static constexpr int kMaxCopies = 5;                   // waves rt = 0, 1; the others 4
    static constexpr int kPages = 1;
    static constexpr int kQBytes = 4 * 18 * 64 * 16;        // [rt][s][lane] x 16 B
    __device__ static int swz(int n) { return n & 7; }
};

template <int KVT>
constexpr int mla_lds_bytes()
{
    return (MlaCfg<KVT>::kQBytes + 4 * MlaCfg<KVT>::kPages * 16 * MlaCfg<KVT>::kRowBytes) > (kMlaObufBytes + 1024)
               ? (MlaCfg<KVT>::kQBytes + 4 * MlaCfg<KVT>::kPages * 16 * MlaCfg<KVT>::kRowBytes)
               : (kMlaObufBytes + 1024);
}

struct MlaState {
    floatx4_t o[32];     // O^T tiles of the wave's row tile (dim mapping: see the epilogue)
    float m;             // running max (log2-scaled logits) of the lane's row
    float l;             // the lane's partial sum of 2^(x - m)
};

// Per-lane LDS byte offsets of one piece's page loop, so the loop adds only
// immediates to them.  FP8: K operand rows k0 / k1 (the two 16-byte halves of
// chunk 0 of lane (n, j); chunk c adds 128 c because the swizzle only touches
// the low two slot bits), Q operands q (block (rt, c, part) adds
// (2 c + part) 2048), V reads v0 / v1 (transposed reads of even / odd index
// p, see mla_pv_f8; read p adds 64 (p >> 1)).  bf16: K slices of even / odd
// index k0 / k1 (slice s adds 64 s), Q q (slice s adds 1024 s), V reads
// v0 .. v3 (transposed reads of tiles T with T % 4 = 0 .. 3, see mla_pv_bf16;
// tile T adds 128 (T >> 2)).
struct MlaLane {
    uint32_t k0, k1, k0b, k1b, q, v0, v1, v2, v3;
};

template <int KVT>
__device__ __forceinline__ MlaLane mla_lane(int rt, int lane)
{
    const int n = lane & 15, j = lane >> 4;
    const int sw = MlaCfg<KVT>::swz(n);
    MlaLane a;
    if constexpr (KVT == kKvFp8) {
        // the second page of a step is stored with the swizzle swz(n) ^ 2
        a.k0 = (uint32_t)(kMlaDim * n + 16 * ((2 * j) ^ sw));
        a.k1 = (uint32_t)(kMlaDim * n + 16 * ((2 * j + 1) ^ sw));
        a.k0b = (uint32_t)(kMlaDim * n + 16 * ((2 * j) ^ sw ^ 2));
        a.k1b = (uint32_t)(kMlaDim * n + 16 * ((2 * j + 1) ^ sw ^ 2));
        a.q = (uint32_t)(rt * 5 * 2 * 2048 + lane * 16);
        // transposed V reads (see mla_pv_f8): lane l addresses key row
        // 4 (l >> 4) + ((l >> 1) & 3) of page (l >> 3) & 1 of the step, dims
        // 16 T + 8 (l & 1) .. + 7
        const int tn = 4 * j + ((lane >> 1) & 3), tp = (lane >> 3) & 1, th = lane & 1;
        const int tw = MlaCfg<kKvFp8>::swz(tn) ^ (2 * tp);
        const uint32_t row = (uint32_t)(tp * 16 * kMlaDim + kMlaDim * tn + 8 * th);
        a.v0 = row + 16 * (0 ^ tw);                                          // T % 4 = 0
        a.v1 = row + 16 * (1 ^ tw);
        a.v2 = row + 16 * (2 ^ tw);
        a.v3 = row + 16 * (3 ^ tw);
    } else {
        const int lo = (j ^ sw) & 3, hi = sw & 4;          // slot 4 s + j -> 4 s +- hi + lo
        a.k0 = (uint32_t)(2 * kMlaDim * n + 16 * (hi + lo));
        a.k1 = (uint32_t)(2 * kMlaDim * n + 16 * (lo - hi));
        a.k0b = a.k1b = 0;
        a.q = (uint32_t)(rt * 18 * 1024 + lane * 16);
        // transposed V reads (see mla_pv_bf16): lane l addresses key row
        // 4 (l >> 4) + ((l >> 2) & 3), dims 16 T + 4 (l & 3) .. + 3
        const int tn = 4 * j + ((lane >> 2) & 3), ta = lane & 3;
        const int tw = MlaCfg<kKvBf16>::swz(tn);
        const uint32_t row = (uint32_t)(2 * kMlaDim * tn + 8 * (ta & 1));
        a.v0 = row + 16 * ((0 + (ta >> 1)) ^ tw);                         // T % 4 = 0
        a.v1 = row + 16 * ((2 + (ta >> 1)) ^ tw);                         // T % 4 = 1
        a.v2 = row + 16 * ((4 + (ta >> 1)) ^ tw);                         // T % 4 = 2
        a.v3 = row + 16 * ((6 + (ta >> 1)) ^ tw);                         // T % 4 = 3
    }
    return a;
}

// S^T (16 keys x 16 rows of row tile rt) of the two pages of a step, FP8: 5
// chunks of 128 dims (the last one half empty: dims 576..639 are zero in Q),
// Q as the exact hi + lo pair, each Q operand used for both pages.  The hi
// operands come from registers (qhi[c], loaded once per piece), the lo ones
// from LDS: with both read from LDS in every step the kernel ran 2-5 % slower
// (LDS bandwidth; register room is left for one of the two).
__device__ __forceinline__ void mla_qk_f8(floatx4_t (&S)[2], const unsigned char *stage, const unsigned char *qlds,
                                          const MlaLane &ad, int lane, const intx8_t (&qhi)[5])
{
    constexpr int kPageBytes = 16 * kMlaDim;
    const int j = lane >> 4;
    floatx4_t Sp[2][2];                                // [page][hi, lo]: 4 independent chains
#pragma unroll
    for (int a = 0; a < 2; ++a)
        Sp[a][0] = Sp[a][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 5; ++c) {
        // chunk 4 of lanes j >= 2 would be dims 576..: they read chunk 4 of
        // lane j - 2 (inside the row).  Their Q operand is zero, so a key
        // adds nothing there unless its row holds a NaN, and then the lanes
        // j - 2 that own those dims make the same logit NaN anyway.
        const uint32_t fix = c == 4 ? (uint32_t)((j >> 1) << 6) : 0u;
        intx8_t kop[2];
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
            const unsigned char *base = stage + pg * kPageBytes - fix + 128 * c;
            const uint4 a = *reinterpret_cast<const uint4 *>(base + (pg ? ad.k0b : ad.k0));
            const uint4 b = *reinterpret_cast<const uint4 *>(base + (pg ? ad.k1b : ad.k1));
            kop[pg] = intx8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
        }
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            intx8_t qop;
            if (part == 0) {
                qop = qhi[c];
            } else {
                const uint4 *qp = reinterpret_cast<const uint4 *>(qlds + ad.q + (2 * c + part) * 2048);
                const uint4 q0 = qp[0], q1 = qp[64];
                qop = intx8_t{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w,
                              (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
            }
            Sp[0][part] = mfma16_f8(kop[0], qop, Sp[0][part]);
            Sp[1][part] = mfma16_f8(kop[1], qop, Sp[1][part]);
        }
        asm volatile("" ::: "memory");                 // one chunk's operands live at a time
    }
    S[0] = Sp[0][0] + Sp[0][1];
    S[1] = Sp[1][0] + Sp[1][1];
}

// The same for a bf16 cache: 18 slices of 32 dims on v_mfma_f32_16x16x32_bf16.
// The Q operands of the first kMlaQRegBf16 slices come from registers (qreg,
// loaded once per piece), the rest from LDS: the registers left beside the
// accumulators hold 12 slices, and fewer LDS reads per step made the bf16 MLA
// kernel 4-5 % faster (8 slices: 3 %, 14: 2 %).
constexpr int kMlaQRegBf16 = 12;
__device__ __forceinline__ floatx4_t mla_qk_bf16(const unsigned char *stage, const unsigned char *qlds,
                                                 const MlaLane &ad, const bf16x8_t (&qreg)[kMlaQRegBf16])
{
    floatx4_t Sp[3];                                   // 3 independent chains
#pragma unroll
    for (int a = 0; a < 3; ++a)
        Sp[a] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 18; ++s) {
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t *>(stage + ((s & 1) ? ad.k1 : ad.k0) + 64 * s);
        const bf16x8_t qop = s < kMlaQRegBf16 ? qreg[s < kMlaQRegBf16 ? s : 0]      // (index kept in range)
                                              : *reinterpret_cast<const bf16x8_t *>(qlds + ad.q + 1024 * s);
        Sp[s % 3] = mfma16(kop, qop, Sp[s % 3]);
    }
    return (Sp[0] + Sp[1]) + Sp[2];
}

// Online softmax of one page for the wave's row tile (lane: row l%16, keys
// key0 + 4 (l/16) + e); same rules as softmax_step1.  Returns the P^T operand.
__device__ __forceinline__ shortx4_t mla_softmax(MlaState &st, const floatx4_t &S, int limit, int key0, float c,
                                                 int lane, bool masked)
{
    const int j = lane >> 4;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v = S[e] * c;
        x[e] = (masked && key0 + 4 * j + e > limit) ? -INFINITY : v;
    }
    const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__any(lmax > st.m + kTau)) {
        float t = fmaxf(lmax, __shfl_xor(lmax, 16));
        t = fmaxf(t, __shfl_xor(t, 32));
        const bool need = t > st.m + kTau;
        const float alpha = need ? exp2_fast(st.m - t) : 1.0f;
        st.m = need ? t : st.m;
        st.l *= alpha;
#pragma unroll
        for (int T = 0; T < 32; ++T)
            st.o[T] *= alpha;
    }
    const float mref = st.m == -INFINITY ? 0.0f : st.m;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pv[e] = exp2_fast(x[e] - mref);
    st.l += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    return __builtin_bit_cast(shortx4_t, make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])));
}

// Online softmax of the two pages of an FP8 step (lane: row l%16, keys
// key0 + 4 (l/16) + e of page 0 and key0 + 16 + 4 (l/16) + e of page 1; the
// second page is absent when !hasb).  Returns the B operand of the 32-key PV
// MFMA: K position 8 j + e is key 4 j + e of page 0, 8 j + 4 + e the same key
// of page 1 (the V operands use the same order).
__device__ __forceinline__ bf16x8_t mla_softmax2(MlaState &st, const floatx4_t (&S)[2], int limit, int key0,
                                                 float c, int lane, bool masked, bool hasb)
{
    const int j = lane >> 4;
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = S[0][e] * c;
        x[4 + e] = S[1][e] * c;
    }
    if (masked) {                                      // uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = key0 + 4 * j + e > limit ? -INFINITY : x[e];
            x[4 + e] = (!hasb || key0 + 16 + 4 * j + e > limit) ? -INFINITY : x[4 + e];
        }
    }
    float lmax = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e)
        lmax = fmaxf(lmax, x[e]);
    if (__any(lmax > st.m + kTau)) {
        float t = fmaxf(lmax, __shfl_xor(lmax, 16));
        t = fmaxf(t, __shfl_xor(t, 32));
        const bool need = t > st.m + kTau;
        const float alpha = need ? exp2_fast(st.m - t) : 1.0f;
        st.m = need ? t : st.m;
        st.l *= alpha;
#pragma unroll
        for (int T = 0; T < 32; ++T)
            st.o[T] *= alpha;
    }
    const float mref = st.m == -INFINITY ? 0.0f : st.m;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        pv[e] = exp2_fast(x[e] - mref);
    st.l += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                   pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])));
}

// LDS transposed read (ds_read_b64_tr_b8).  Measured lane rule on gfx950:
// within each group of 16 lanes, output lane 16 g + 8 h + b receives as its
// byte i byte b of the 8 bytes addressed by input lane 16 g + 2 i + h.
__device__ __forceinline__ uint2 lds_read_tr8(const unsigned char *p)
{
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_t *)p);
    return make_uint2((uint32_t)r.x, (uint32_t)r.y);
}

// O^T += V^T P^T over the latent of the two pages of an FP8 step, on the
// 32-key bf16 MFMA.  Read T (0..31) is one transposed read: input lane l
// addresses the 8 dims 16 T + 8 (l & 1) .. + 7 of key row 4 (l >> 4) +
// ((l >> 1) & 3) of page (l >> 3) & 1.  Output lane (n, j) then holds dim
// 16 T + n of keys 4 j .. 4 j + 3 of page 0 (bytes 0..3) and page 1 (bytes
// 4..7): the A operand of tile T in the K order of mla_softmax2, converted
// exactly to bf16, with no byte shuffles.
// Key rows at or past the end of the sequence or of the piece (poisoned or
// stale) have been zeroed in the stage (mla_zero_rows), so their zero weights
// meet zero values.
__device__ __forceinline__ void mla_pv_f8(MlaState &st, const unsigned char *stage, const bf16x8_t &pop,
                                          const MlaLane &ad)
{
#pragma unroll
    for (int T = 0; T < 32; ++T) {
        const uint32_t b = (T & 3) == 0 ? ad.v0 : (T & 3) == 1 ? ad.v1 : (T & 3) == 2 ? ad.v2 : ad.v3;
        const uint2 r = lds_read_tr8(stage + b + 64 * (T >> 2));
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(fp8x2_lo_to_bf16x2(r.x), fp8x2_hi_to_bf16x2(r.x),
                                                                  fp8x2_lo_to_bf16x2(r.y), fp8x2_hi_to_bf16x2(r.y)));
        st.o[T] = mfma16(a, pop, st.o[T]);
    }
}

__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char *p)
{
    typedef short v4s_t __attribute__((ext_vector_type(4)));
    const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t *)p);
    return __builtin_bit_cast(uint2, r);
}

// The same for a bf16 cache, with ds_read_b64_tr_b16 (measured lane rule:
// within each group of 16 lanes, output lane 16 g + 4 a + b receives as its
// element i element b of the 4 addressed by input lane 16 g + 4 i + a).
// Input lane l addresses dims 16 T + 4 (l & 3) .. + 3 of key row
// 4 (l >> 4) + ((l >> 2) & 3), so output lane (n, j) holds dim 16 T + n of
// keys 4 j .. 4 j + 3: the A operand of tile T as read, one read per tile.
// Key rows past the end have been zeroed in the stage, as for FP8.
__device__ __forceinline__ void mla_pv_bf16(MlaState &st, const unsigned char *stage, const shortx4_t &pop,
                                            const MlaLane &ad)
{
#pragma unroll
    for (int T = 0; T < 32; ++T) {
        const uint32_t b = (T & 3) == 0 ? ad.v0 : (T & 3) == 1 ? ad.v1 : (T & 3) == 2 ? ad.v2 : ad.v3;
        const uint2 r = lds_read_tr16(stage + b + 128 * (T >> 2));
        st.o[T] = mfma16k16(__builtin_bit_cast(shortx4_t, r), pop, st.o[T]);
    }
}

// Zeroes, in a ring stage of np pages of 16 rows, the rows n >= nv[pg] of page
// pg (whole rows, every slot).  Each wave that reads the stage does this itself
// on its own schedule: every write is a zero, so no order between the waves
// matters, and a wave's own writes precede its reads.
template <int ROW>
__device__ __forceinline__ void mla_zero_rows(unsigned char *stage, int np, int nv0, int nv1, int lane)
{
    constexpr int kSlots = ROW / 16;                   // 16-byte slots per row
    for (int i = lane; i < np * 16 * kSlots; i += 64) {
        const int pg = i / (16 * kSlots), rem = i - pg * 16 * kSlots;
        const int n = rem / kSlots;
        if (n >= (pg ? nv1 : nv0))
            *reinterpret_cast<uint4 *>(stage + pg * 16 * ROW + rem * 16) = make_uint4(0, 0, 0, 0);
    }
}

// Split-KV main kernel for absorbed MLA.  Same work split (stream-K over the
// pages of all sequences), partials and whole-piece output rules as the GQA
// kernels, with 512-wide rows of O.
template <int KVT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void va_mla_split_kernel(SplitParams p)
{
    using C = MlaCfg<KVT>;
    constexpr int kPageBytes = 16 * C::kRowBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[mla_lds_bytes<KVT>()];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int rt = wave & 3;                           // row tile
    const int kg = wave >> 2;                          // key group
    // Each SIMD holds one wave of each key group (wave w runs on SIMD w % 4),
    // and both run the same QK -> softmax -> PV order behind one barrier per
    // step.  Key group 0 issues at a higher priority, so its waves run ahead
    // and the two waves of a SIMD drift into different phases: one wave's
    // matrix work then overlaps the other's vector and LDS work (measured 8 %
    // to 10 % faster with an FP8 cache, 2 % with bf16; bit-identical output).
    if (kg == 0)
        __builtin_amdgcn_s_setprio(3);
    const int w = blockIdx.x;
    const int G = 1 << p.log2g;

    Share sh = locate(p, w, lane, w == 0 && wave == 0);
    sh.n_eff = uniform(sh.n_eff);
    sh.s = uniform(sh.s);
    sh.e = uniform(sh.e);
    sh.bg = uniform(sh.bg);
    sh.base = uniform(sh.base);
    if (w >= sh.n_eff)
        return;                                        // uniform over the workgroup

    // (vector loads here: with scalar ones the compiler schedules the PV's
    // transposed reads one at a time, measured 4-8 % slower)
    const float kd = p.kdesc ? p.kdesc[0] : 1.0f;
    const float vd = p.vdesc ? p.vdesc[0] : 1.0f;
    const float c = p.scale_log2 * kd;
    unsigned char *qlds = lds;
    constexpr int PP = C::kPages;                      // pages per step of a key group
    unsigned char *ring = lds + C::kQBytes + kg * 2 * PP * kPageBytes;
    const uint32_t ring_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(ring));
    const uint32_t lds_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(lds));
    const int64_t page_bytes = (int64_t)kPage * C::kRowBytes;
    const int ncp = uniform((C::kCopies - rt + 3) / 4);     // copies this wave issues per page

    const int bh = p.num_seqs;                             // one kv head
    int s = sh.s, bg = sh.bg, base = sh.base;
    while (s < sh.e && bg < bh) {
        int pl = lane;                                 // opaque per piece (see the FP8 GQA kernel)
        asm volatile("" : "+v"(pl));
        const int b = bg;
        const int q0 = load_uniform(p.cu, b);
        const int lq = checked_q_len(q0, load_uniform(p.cu, b + 1), p.total_q, p.max_q);
        const int lk = load_uniform(p.seqused, b);
        const int cnt = (lq <= 0 || lk <= 0) ? 0 : max(0, min((lk + kPage - 1) / kPage, p.mbps));
        if (cnt == 0) {
            ++bg;
            continue;
        }
        const int ctx = lk - lq;
        const int r0 = s - base;
        const int r1 = min(sh.e, base + cnt) - base;
        const bool whole = (r0 == 0 && r1 == cnt);
        const int p0 = r0;
        const int npg = r1 - r0;                           // pages of the piece
        const int nblk = (npg + PP - 1) / PP;              // steps of PP pages; key group kg
        const int nsteps = (nblk + 1) >> 1;                // takes blocks kg, kg + 2, ... (uniform)
        const int slot = 2 * w + (s != sh.s);           // first or last piece of this workgroup
        const int R = lq * G;
        const bool rows_live = 16 * rt < R;
        const int32_t *btrow = p.bt + (int64_t)b * p.mbps;
        const int64_t maxpage = p.num_blocks - 1;
        auto pages_in = [&](int u) { return max(0, min(PP, npg - PP * u)); };   // pages of block u
        auto issue = [&](int u, int stage) {               // this wave's copies of block u of the piece
#pragma unroll
            for (int pg = 0; pg < PP; ++pg) {
                if (PP * u + pg >= npg)
                    break;                                 // uniform
                int64_t y = load_uniform(btrow, uniform(p0 + PP * u + pg));
                y = y < 0 ? 0 : (y > maxpage ? maxpage : y);
                const uint8_t *a = p.k + y * page_bytes;
                const uint32_t dst = ring_addr + (stage * PP + pg) * kPageBytes;
                int ln = lane;                             // lane offsets rederived per copy (no
                asm volatile("" : "+v"(ln));               // registers held across the page loop)
#pragma unroll
                for (int i = 0; i < C::kMaxCopies; ++i)
                    if (i < ncp) {
                        const int sl = 64 * (rt + 4 * i) + ln; // LDS slot of this lane's 16 bytes
                        const int n = sl / C::kChunks;         // key row; page pg of a step uses swz ^ 2 pg
                        const uint32_t off =
                            (uint32_t)(n * C::kRowBytes + 16 * ((sl - n * C::kChunks) ^ C::swz(n) ^ (2 * pg)));
                        dma16(a, off, dst + 1024 * (rt + 4 * i));
                    }
            }
        };
        auto wait_older = [&](int np) {                    // this wave's copies of the older block
            if (np == 2) {                                 // landed; np pages of the next one may not
                if (ncp == C::kMaxCopies)
                    wait_vmcnt<2 * C::kMaxCopies>();
                else
                    wait_vmcnt<2 * (C::kMaxCopies - 1)>();
            } else if (np == 1) {
                if (ncp == C::kMaxCopies)
                    wait_vmcnt<C::kMaxCopies>();
                else
                    wait_vmcnt<C::kMaxCopies - 1>();
            } else {
                wait_vmcnt<0>();
            }
        };

        // ---- prologue: the first page of each key group; Q operands; the second
        __syncthreads();                                   // previous piece's LDS reads done
        float crow = c;                                    // logit multiplier of this lane's row
        if constexpr (KVT == kKvFp8) {
            if (kg < nblk)
                issue(kg, 0);
            // this wave's row tile, lane (row n, j): dims 128 cc + 32 j .. +32
            const int n = pl & 15, j = pl >> 4;
            const int r = 16 * rt + n;
            const int t = r >> p.log2g;
            const bool live = r < R;
            const uint16_t *qrow = p.q + ((int64_t)(q0 + (live ? t : 0)) * p.hq + (r & (G - 1))) * kMlaDim;
            uint32_t raw[5][16];
#pragma unroll
            for (int cc = 0; cc < 5; ++cc) {
                const bool have = live && (cc < 4 || j < 2);   // dims 576.. do not exist
                const int jj = cc < 4 ? j : (j & 1);           // in-row address for every lane
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint4 v = *reinterpret_cast<const uint4 *>(qrow + 128 * cc + 32 * jj + 8 * i);
                    if (!have)
                        v = make_uint4(0, 0, 0, 0);
                    raw[cc][4 * i] = v.x;
                    raw[cc][4 * i + 1] = v.y;
                    raw[cc][4 * i + 2] = v.z;
                    raw[cc][4 * i + 3] = v.w;
                }
            }
            float amax = 0.f;
#pragma unroll
            for (int cc = 0; cc < 5; ++cc)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[cc][i] << 16)),
                                             fabsf(__builtin_bit_cast(float, raw[cc][i] & 0xFFFF0000u))));
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));          // row max (4 lanes)
            int kx = 0;
            if (amax > 0.f) {
                int e;
                frexpf(amax, &e);
                kx = min(8 - e, 127);
            }
            crow = ldexpf(c, -kx);
            // key group 0 converts chunks 0..2, key group 1 chunks 3..4
#pragma unroll
            for (int cc = 0; cc < 5; ++cc)
                if ((cc < 3) == (kg == 0))
                    convert_q_block<1>(qlds, raw[cc], kx, rt * 5 + cc, pl);
            __syncthreads();                               // Q operands visible
            if (kg + 2 < nblk)
                issue(kg + 2, 1);
        } else {
            // Q operands copied straight in operand order: copy i = rt' * 18 + sl,
            // lane l gets dims 32 sl + 8 (l/16) .. +8 of packed row 16 rt' + l%16
            const uint16_t *qbase = p.q + (int64_t)q0 * p.hq * kMlaDim;
            for (int i = wave; i < 4 * 18; i += 8) {
                const int rr = i / 18, sl = i - rr * 18;
                const int r = 16 * rr + (pl & 15);
                int t = r >> p.log2g;
                t = r < R ? t : 0;
                const uint32_t voff = (uint32_t)(((t * p.hq + (r & (G - 1))) * kMlaDim + 32 * sl + 8 * (pl >> 4)) * 2);
                dma16(qbase, voff, lds_addr + i * 1024);
            }
            if (kg < npg)
                issue(kg, 0);
            if (kg + 2 < npg)
                issue(kg + 2, 1);
            wait_vmcnt<0>();                               // (the loop's barrier publishes Q)
        }

        // O starts at zero only here: an opaque zero keeps the 128 accumulator
        // registers from being set (and held) across the Q conversion above
        float z = 0.f;
        asm volatile("" : "+v"(z));
        MlaState st;
        st.m = -INFINITY;
        st.l = 0.f;
#pragma unroll
        for (int T = 0; T < 32; ++T)
            st.o[T] = floatx4_t{z, z, z, z};
        int limit;
        {
            const int r = 16 * rt + (pl & 15);
            limit = min(ctx + (r >> p.log2g), lk - 1);
        }

        const MlaLane ad = mla_lane<KVT>(rt, pl);          // the loop's LDS offsets: 9 registers
        intx8_t qhi[5];                                    // FP8: hi operands of the row tile
        bf16x8_t qreg[kMlaQRegBf16];                       // bf16: the first Q slices
        for (int t = 0; t < nsteps; ++t) {
            const int k = kg + 2 * t;                      // block of the piece
            if (KVT == kKvFp8 && t == 0)
                wait_older(pages_in(k + 2));               // block k landed (block k + 2 may not)
            else
                wait_vmcnt<0>();
            __syncthreads();                               // the group's copies too; stage t-1 free
            if (KVT == kKvFp8 && t == 0) {                 // the Q operands are visible now
#pragma unroll
                for (int c = 0; c < 5; ++c) {
                    const uint4 *qp = reinterpret_cast<const uint4 *>(qlds + ad.q + (2 * c) * 2048);
                    const uint4 q0 = qp[0], q1 = qp[64];
                    qhi[c] = intx8_t{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w,
                                     (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
                }
            }
            if (KVT == kKvBf16 && t == 0) {
#pragma unroll
                for (int sl = 0; sl < kMlaQRegBf16; ++sl)
                    qreg[sl] = *reinterpret_cast<const bf16x8_t *>(qlds + ad.q + 1024 * sl);
            }
            if (t >= 1 && k + 2 < nblk)
                issue(k + 2, (t + 1) & 1);
            if (k < nblk && rows_live) {
                // other lane-derived values are rederived each step from an
                // opaque lane index: hoisted out of the loop they would hold
                // registers next to the 128 accumulators
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const unsigned char *stage = ring + (t & 1) * PP * kPageBytes;
                const int key0 = (p0 + PP * k) * kPage;
                if constexpr (KVT == kKvFp8) {
                    const bool hasb = PP * k + 1 < npg;            // uniform: the step's second page
                    const bool masked = key0 + 31 > ctx || !hasb;
                    if (key0 + 31 >= lk || !hasb)                  // uniform: rows past the end
                        mla_zero_rows<C::kRowBytes>(ring + (t & 1) * PP * kPageBytes, 2, lk - key0,
                                                    hasb ? lk - key0 - 16 : 0, ln);
                    floatx4_t S[2];
                    mla_qk_f8(S, stage, qlds, ad, ln, qhi);
                    const bf16x8_t pop = mla_softmax2(st, S, limit, key0, crow, ln, masked, hasb);
                    mla_pv_f8(st, stage, pop, ad);
                } else {
                    const bool masked = key0 + 15 > ctx;
                    if (key0 + 15 >= lk)                           // uniform: rows past the end
                        mla_zero_rows<C::kRowBytes>(ring + (t & 1) * kPageBytes, 1, lk - key0, 0, ln);
                    const floatx4_t S = mla_qk_bf16(stage, qlds, ad, qreg);
                    const shortx4_t pop = mla_softmax(st, S, limit, key0, crow, ln, masked);
                    mla_pv_bf16(st, stage, pop, ad);
                }
            }
        }
        wait_vmcnt<0>();

        // ---- epilogue: merge the two key groups, then the final rows or a partial
        st.l += __shfl_xor(st.l, 16);
        st.l += __shfl_xor(st.l, 32);
        __syncthreads();                                   // every wave is past its loop
        float *ml = reinterpret_cast<float *>(lds + kMlaObufBytes);
        unsigned char *obuf = lds;
        {
            const int n = pl & 15, j = pl >> 4;
            const int row = 16 * rt + n;
            if (j == 0) {
                ml[(kg * kMlaRows + row) * 2] = st.m;
                ml[(kg * kMlaRows + row) * 2 + 1] = st.l;
            }
            const float inv = st.l > 0.f ? 1.0f / st.l : 0.f;
            unsigned char *orow = obuf + (size_t)(kg * kMlaRows + row) * 1024;
            if constexpr (KVT == kKvFp8) {                 // tile T: dims 16 T + 4 j .. + 3
#pragma unroll
                for (int T = 0; T < 32; ++T) {
                    const int u = 2 * T + (j >> 1);             // 8-dim unit of the row
                    *reinterpret_cast<uint2 *>(orow + 16 * (u ^ n) + 8 * (j & 1)) =
                        make_uint2(pack_f16x2(st.o[T][0] * inv, st.o[T][1] * inv),
                                   pack_f16x2(st.o[T][2] * inv, st.o[T][3] * inv));
                }
            } else {                                       // the same mapping, bf16 units
#pragma unroll
                for (int T = 0; T < 32; ++T) {
                    const int u = 2 * T + (j >> 1);
                    *reinterpret_cast<uint2 *>(orow + 16 * (u ^ n) + 8 * (j & 1)) =
                        make_uint2(pack_bf16x2(st.o[T][0] * inv, st.o[T][1] * inv),
                                   pack_bf16x2(st.o[T][2] * inv, st.o[T][3] * inv));
                }
            }
        }
        __syncthreads();
        const int tid = opaque_tid();
        const int nrows = min(R, kMlaRows);
        for (int it = tid; it < nrows * 64; it += 512) {
            const int r = it >> 6, u = it & 63;            // row, 8-dim unit
            float M = -INFINITY;
            float mk[2], lkk[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                mk[k2] = ml[(k2 * kMlaRows + r) * 2];
                lkk[k2] = ml[(k2 * kMlaRows + r) * 2 + 1];
                M = fmaxf(M, lkk[k2] > 0.f ? mk[k2] : -INFINITY);
            }
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float W = 0.f;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const float wk = lkk[k2] > 0.f ? lkk[k2] * exp2_fast(mk[k2] - M) : 0.f;
                W += wk;
                const uint4 v = *reinterpret_cast<const uint4 *>(obuf + (size_t)(k2 * kMlaRows + r) * 1024 +
                                                                 16 * (u ^ (r & 15)));
                acc[0] += wk * xlo<KVT>(v.x);
                acc[1] += wk * xhi<KVT>(v.x);
                acc[2] += wk * xlo<KVT>(v.y);
                acc[3] += wk * xhi<KVT>(v.y);
                acc[4] += wk * xlo<KVT>(v.z);
                acc[5] += wk * xhi<KVT>(v.z);
                acc[6] += wk * xlo<KVT>(v.w);
                acc[7] += wk * xhi<KVT>(v.w);
            }
            const int t = r >> p.log2g, hh = r & (G - 1);
            if (whole) {
                const float sc = W > 0.f ? vd / W : 0.f;
                uint4 o;
                o.x = pack_bf16x2(acc[0] * sc, acc[1] * sc);
                o.y = pack_bf16x2(acc[2] * sc, acc[3] * sc);
                o.z = pack_bf16x2(acc[4] * sc, acc[5] * sc);
                o.w = pack_bf16x2(acc[6] * sc, acc[7] * sc);
                *reinterpret_cast<uint4 *>(p.out + ((int64_t)(q0 + t) * p.hq + hh) * kMlaDv + 8 * u) = o;
            } else {
                const float sc = W > 0.f ? 1.0f / W : 0.f;
                const int64_t sr = ((int64_t)slot * kMlaRows + r) * kMlaDv + 8 * u;
                if constexpr (KVT == kKvFp8) {
                    uint4 o;
                    o.x = pack_f16x2(acc[0] * sc, acc[1] * sc);
                    o.y = pack_f16x2(acc[2] * sc, acc[3] * sc);
                    o.z = pack_f16x2(acc[4] * sc, acc[5] * sc);
                    o.w = pack_f16x2(acc[6] * sc, acc[7] * sc);
                    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.ws_o) + sr) = o;
                } else {
                    float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(p.ws_o) + sr);
                    dst[0] = make_float4(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc);
                    dst[1] = make_float4(acc[4] * sc, acc[5] * sc, acc[6] * sc, acc[7] * sc);
                }
                if (u == 0)
                    p.ws_lse[(int64_t)slot * kMlaRows + r] = W > 0.f ? M + __log2f(W) : -INFINITY;
            }
        }

        s = base + r1;
        base += cnt;
        ++bg;
    }
}

// Segment reduce.  One workgroup = NT / (DV / 4) consecutive heads of one
// query token: one head of a 256-wide row (NT = 64), two of a 512-wide MLA row
// (NT = 256); DV / 4 threads per row, 4 dims each.  One head per workgroup
// spreads the partial reads over more CUs than four did (high-concurrency and
// shape-sweep calls 0.2-0.4 us faster).  The partials of a row are read in
// chunks of 16 slots with all loads of a chunk issued before any is used.
template <bool kHalf>
__device__ __forceinline__ float4 load_partial4(const void *base, int64_t idx)
{
    if constexpr (kHalf) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
        return make_float4(f16_lo(u.x), f16_hi(u.x), f16_lo(u.y), f16_hi(u.y));
    } else {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    }
}

constexpr int kMergeThreadsGqa = 64;                // merge workgroup, 256-wide rows

template <bool kHalf, int DV, int NT>
__global__ __launch_bounds__(NT) void va_merge_kernel(MergeParams p)
{
    constexpr int kChunk = 16;
    constexpr int kTpr = DV / 4;                        // threads per row
    constexpr int kHpb = NT / kTpr;                     // heads per workgroup
    const int gq = (1 << p.log2g) / kHpb;               // workgroups per (token, group)
    int idx = blockIdx.x;
    const int hq4 = idx % gq;
    idx /= gq;
    const int t = idx % p.max_q;
    const int bg = idx / p.max_q;
    const int b = bg / p.hkv;
    const int g = bg - b * p.hkv;
    const int bh = p.num_seqs * p.hkv;
    // every metadata word is loaded before any is used: one round trip
    const int q0 = load_uniform(p.cu, b);
    const int q1 = load_uniform(p.cu, b + 1);
    const int s = load_uniform(p.ws_prefix, bg);
    const int e = load_uniform(p.ws_prefix, bg + 1);
    const int cs = load_uniform(p.ws_cost, bg);
    const int ce = load_uniform(p.ws_cost, bg + 1);
    const int ctot = load_uniform(p.ws_cost, bh);
    const int nw = load_uniform(p.ws_meta, 0);
    asm volatile("" :: "s"(q0), "s"(q1), "s"(s), "s"(e), "s"(cs), "s"(ce), "s"(ctot), "s"(nw));   // one round trip
    const int64_t n = nw;
    const int lq = checked_q_len(q0, q1, p.total_q, p.max_q);
    if (t >= lq || e <= s || ctot <= 0)
        return;
    // The split of locate() in cost positions: the pair's pages occupy cost
    // positions [ce - (e - s), ce); workgroup w covers [w T / n, (w + 1) T / n).
    const int64_t x0 = ce - (e - s);                   // cost position of the pair's first page
    const int w0 = (int)(((x0 + 1) * n - 1) / ctot);
    const int w1 = (int)(((int64_t)ce * n - 1) / ctot);
    if (w0 == w1)
        return;                                        // written by the main kernel
    const int h = hq4 * kHpb + threadIdx.x / kTpr;
    const int row = (t << p.log2g) + h;
    const int d = (threadIdx.x % kTpr) * 4;
    // Slots of the pieces: workgroup w0 holds this pair as its first piece
    // (slot 2 w0) if its range starts inside the pair's costs, else as its last
    // (2 w0 + 1); every later workgroup w holds it as its first piece (2 w).
    const int first0 = cs > (int)(((int64_t)w0 * ctot) / n) ? 1 : 0;
    const int ns = w1 - w0 + 1;
    auto slot_of = [&](int si) -> int64_t { return si == 0 ? 2 * w0 + first0 : 2 * (w0 + si); };

    // One pass over the slots, kChunk at a time with every load of a chunk in
    // flight; the running max moves per chunk (the sum is rescaled then).
    float mx = -INFINITY;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int c0 = 0; c0 < ns; c0 += kChunk) {
        float l[kChunk];
        float4 v[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {                 // unconditional loads (a slot past the
            const int64_t sl = slot_of(min(c0 + i, ns - 1));  // end re-reads the last one), then masked
            l[i] = p.ws_lse[sl * p.rows_max + row];
            v[i] = load_partial4<kHalf>(p.ws_o, (sl * p.rows_max + row) * DV + d);
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            if (c0 + i >= ns)
                l[i] = -INFINITY;
        float mc = l[0];
#pragma unroll
        for (int i = 1; i < kChunk; ++i)
            mc = fmaxf(mc, l[i]);
        if (mc > mx) {
            const float f = mx == -INFINITY ? 0.f : exp2_fast(mx - mc);
            den *= f;
            acc.x *= f;
            acc.y *= f;
            acc.z *= f;
            acc.w *= f;
            mx = mc;
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const float f = l[i] == -INFINITY ? 0.f : exp2_fast(l[i] - mx);
            den += f;
            acc.x += f * v[i].x;
            acc.y += f * v[i].y;
            acc.z += f * v[i].z;
            acc.w += f * v[i].w;
        }
    }
    if (p.sinks) {                                     // the sink joins the denominator once
        const float sk = p.sinks[g * (1 << p.log2g) + h] * 1.4426950408889634f;
        const float mm = fmaxf(mx, sk);
        const float f = den > 0.f ? exp2_fast(mx - mm) : 0.f;
        den = den * f + exp2_fast(sk - mm);
        acc.x *= f;
        acc.y *= f;
        acc.z *= f;
        acc.w *= f;
    }
    const float vd = load_descale(p.vdesc);
    const float inv = den > 0.f ? vd / den : 0.f;
    uint2 pk;
    pk.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    pk.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    const int G = 1 << p.log2g;
    *reinterpret_cast<uint2 *>(p.out + ((int64_t)(q0 + t) * p.hq + g * G + h) * DV + d) = pk;
}

// Draft-extend metadata: one thread per block-table entry (b, page).  Page pg
// of sequence b is the pool page of its token pg * page_size, whose slot is
// kv_indices[kv_indptr[b] + pg * page_size]; the page-0 thread also writes
// seqused_k[b] = kv_indptr[b + 1] - kv_indptr[b].
__global__ __launch_bounds__(kThreads) void va_spec_block_table_kernel(const int32_t *indptr, const int32_t *indices,
                                                                       int32_t num_seqs, int32_t page_size,
                                                                       int32_t mbps, int32_t *bt, int32_t *seqused)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)num_seqs * mbps)
        return;
    const int b = (int)(i / mbps);
    const int pg = (int)(i - (int64_t)b * mbps);
    const int64_t t0 = indptr[b];
    const int64_t n = (int64_t)indptr[b + 1] - t0;
    if (pg == 0)
        seqused[b] = (int32_t)n;
    const int64_t tok = (int64_t)pg * page_size;
    bt[i] = tok < n ? indices[t0 + tok] / page_size : 0;
}

// Streaming ceiling (diagnostic): the copy path of the FP8 paged kernel with
// nothing else.  Each wave takes an equal contiguous share of a list of 4 KiB
// pages and copies them in that order into a ring of DEPTH 4 KiB slots of its
// own LDS region (40 KiB, as the FP8 kernel's ring) with the same
// global_load_lds_dwordx4 ... nt copies, keeping DEPTH pages in flight.  When
// a slot is reused, the first dword of the page that landed there is added to
// the wave's sum (so the copies are checked, not only issued); sums[wave]
// holds the total.  Pages are pool + 4096 * pages[i], with the index clamped
// to the pool.
template <int DEPTH>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void va_stream_pages_kernel(const uint8_t *pool, int64_t pool_pages, const int32_t *pages, int64_t npages,
                            uint32_t *sums)
{
    static_assert(DEPTH >= 1 && DEPTH <= 10, "ring of at most 10 slots");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * 10 * 4096];
    const int lane = threadIdx.x & 63;
    const int wv = uniform(threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wv;
    const int64_t a = (gw * npages) / nw, b = ((gw + 1) * npages) / nw;
    unsigned char *ring = lds + wv * 10 * 4096;
    const uint32_t ring_addr = uniform((int)(uint32_t)reinterpret_cast<uintptr_t>(ring));
    uint32_t sum = 0;
    for (int64_t i = a; i < b; ++i) {
        const int slot = (int)((i - a) % DEPTH);
        if (i - a >= DEPTH) {
            wait_vmcnt<4 * (DEPTH - 1)>();              // the page that used this slot landed
            sum += *reinterpret_cast<const uint32_t *>(ring + slot * 4096);
        }
        const int64_t pg = min(max((int64_t)load_uniform(pages, i), (int64_t)0), pool_pages - 1);   // clamped
        const uint8_t *src = pool + pg * 4096;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            dma16(src, (uint32_t)(1024 * x + 16 * lane), ring_addr + (uint32_t)(slot * 4096 + 1024 * x));
    }
    wait_vmcnt<0>();
    const int64_t done = b - a;
    for (int64_t i = max(a, b - DEPTH); i < b; ++i)
        sum += *reinterpret_cast<const uint32_t *>(ring + (int)((i - a) % DEPTH) * 4096);
    if (lane == 0)
        sums[gw] = done > 0 ? sum : 0u;
}

__global__ __launch_bounds__(kThreads) void va_fp8_to_bf16_kernel(const uint8_t *in, uint16_t *out, int64_t n)
{
    const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (i >= n)
        return;
    uint32_t w = 0;
    for (int k = 0; k < 4 && i + k < n; ++k)
        w |= (uint32_t)in[i + k] << (8 * k);
    const uint32_t lo = fp8x2_lo_to_bf16x2(w);
    const uint32_t hi = fp8x2_hi_to_bf16x2(w);
    const uint16_t r[4] = {(uint16_t)(lo & 0xFFFF), (uint16_t)(lo >> 16), (uint16_t)(hi & 0xFFFF),
                           (uint16_t)(hi >> 16)};
    for (int k = 0; k < 4 && i + k < n; ++k)
        out[i + k] = r[k];
}

// Validate mode: checks of one call's device metadata.  One thread per
// block-table entry (b, page).  The page-0 thread of a sequence checks its
// lengths; every thread checks its own entry if the sequence reads it.
// res[0] collects the VA_BAD_* bits, res[1] the smallest offending sequence
// (va_validate_init_kernel first sets num_seqs there).
struct ValidateParams {
    const int32_t *bt;
    const int32_t *cu;
    const int32_t *seqused;
    int32_t *res;
    int32_t num_seqs, mbps, max_q, max_k, window_left;
    int64_t total_q, num_blocks;
};

__global__ __launch_bounds__(64) void va_validate_init_kernel(int32_t *res, int32_t num_seqs)
{
    if (threadIdx.x == 0) {
        res[0] = 0;
        res[1] = num_seqs;
    }
}

__global__ __launch_bounds__(kThreads) void va_validate_kernel(ValidateParams p)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)p.num_seqs * p.mbps)
        return;
    const int b = (int)(i / p.mbps);
    const int pg = (int)(i - (int64_t)b * p.mbps);
    const int64_t q0 = p.cu[b], q1 = p.cu[b + 1];
    const int64_t lk = p.seqused[b];
    const bool cu_ok = !(b == 0 && q0 != 0) && q1 >= q0 && q1 <= p.total_q;
    const int64_t lq = cu_ok ? q1 - q0 : 0;
    int bad = 0;
    if (pg == 0) {
        if (!cu_ok)
            bad |= VA_BAD_CU_SEQLENS_Q;
        if (lq > p.max_q)
            bad |= VA_BAD_Q_LEN;
        if (lk < 0 || lk > p.max_k)
            bad |= VA_BAD_SEQUSED_K;
        if (lq > lk)
            bad |= VA_BAD_Q_GT_K;
    }
    // entries read: the pages of keys first .. lk - 1 (first = lk - lq -
    // window_left with a window, else 0) inside the block-table row
    const int64_t first = p.window_left < 0 ? 0 : max((int64_t)0, lk - lq - p.window_left) / kPage;
    if (lk > 0 && pg >= first && (int64_t)pg * kPage < lk) {
        const int32_t page = p.bt[i];
        if (page < 0 || page >= p.num_blocks)
            bad |= VA_BAD_PAGE;
    }
    if (bad) {
        atomicOr(p.res, bad);
        atomicMin(p.res + 1, b);
    }
}

// ------------------------------------------------------------------ host --

// A split-KV kernel: every one takes a single SplitParams argument.  All are
// launched through hipExtLaunchKernel, whose optional start / stop events take
// the timestamps of the dispatch itself (va_run_timed); without events it is
// an ordinary launch.
struct SplitKernel {
    const void *fn;
    int threads;
};

template <typename K>
SplitKernel kref(K *fn, int threads)
{
    return SplitKernel{reinterpret_cast<const void *>(fn), threads};
}

template <int RTW, bool CAP, bool TOK>
SplitKernel pick_w8(bool fp8)
{
    return fp8 ? kref(&va_split_kv_fp8_w8_kernel<RTW, CAP, TOK>, 512)
               : kref(&va_split_kv_bf16_w8_kernel<RTW, CAP, TOK>, 512);
}

template <bool CAP>
SplitKernel pick_fp8_w4(int row_tiles)
{
    switch (row_tiles) {
    case 1: return kref(&va_split_kv_fp8_w4_kernel<1, CAP>, 256);
    case 2: return kref(&va_split_kv_fp8_w4_kernel<2, CAP>, 256);
    case 3: return kref(&va_split_kv_fp8_w4_kernel<3, CAP>, 256);
    default: return kref(&va_split_kv_fp8_w4_kernel<4, CAP>, 256);
    }
}

template <int RTW, bool CAP>
SplitKernel pick_layout(bool fp8, bool tok)
{
    return tok ? pick_w8<RTW, CAP, true>(fp8) : pick_w8<RTW, CAP, false>(fp8);
}

// Row tiles needed -> kernel.  A paged FP8 cache runs the one-wave-per-SIMD
// kernel with exactly the row tiles needed.  The others use two row groups of
// RTW row tiles: one or two row tiles take RTW = 1, three or four RTW = 2 (a
// wave's O^T accumulators stay at 128 registers).  Then KV dtype, softcap,
// layout; absorbed MLA has its own kernel.
SplitKernel select_kernel(int row_tiles, bool fp8, bool cap, bool tok, bool mla, bool w4)
{
    if (mla)
        return fp8 ? kref(&va_mla_split_kernel<kKvFp8>, 512) : kref(&va_mla_split_kernel<kKvBf16>, 512);
    if (fp8 && !tok && w4)
        return cap ? pick_fp8_w4<true>(row_tiles) : pick_fp8_w4<false>(row_tiles);
    if (row_tiles <= 2)
        return cap ? pick_layout<1, true>(fp8, tok) : pick_layout<1, false>(fp8, tok);
    return cap ? pick_layout<2, true>(fp8, tok) : pick_layout<2, false>(fp8, tok);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

struct va_plan_s {
    va_problem prob;
    int log2g;
    int rt;             // row tiles the packed rows need (selects the kernel variant)
    int grid;           // split-KV workgroups
    int min_pages;
    int rows_max;
    int64_t slots;
    int32_t mbps;       // pages per sequence bound: the block-table row, or (prefix + extend)
                        // ceil(max_seqlen_k / 16)
    bool mla;           // absorbed MLA: 576-wide rows, 512-wide values (va_mla_split_kernel)
    bool fp8_w4;        // FP8 paged GQA on the one-wave-per-SIMD kernel
    size_t off_prefix, off_cost, off_lse, off_o, ws_bytes;
    int32_t piece_cost;
    bool debug;         // VA_DEBUG set at va_plan: validate mode and a plan dump on stderr
};

namespace {

bool debug_env()
{
    const char *e = getenv("VA_DEBUG");
    return e && e[0] && strcmp(e, "0") != 0;
}

va_status enqueue_validate(const va_plan_s *plan, const int32_t *block_table, const int32_t *cu_seqlens_q,
                           const int32_t *seqused_k, int32_t *result, hipStream_t s)
{
    const va_problem &pr = plan->prob;
    ValidateParams vp;
    vp.bt = block_table;
    vp.cu = cu_seqlens_q;
    vp.seqused = seqused_k;
    vp.res = result;
    vp.num_seqs = pr.num_seqs;
    vp.mbps = pr.max_blocks_per_seq;
    vp.max_q = pr.max_seqlen_q;
    vp.max_k = pr.max_seqlen_k;
    vp.window_left = pr.window_left;
    vp.total_q = pr.total_q;
    vp.num_blocks = pr.num_blocks;
    const int64_t blocks = ((int64_t)pr.num_seqs * pr.max_blocks_per_seq + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(va_validate_init_kernel, dim3(1), dim3(64), 0, s, result, pr.num_seqs);
    hipLaunchKernelGGL(va_validate_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, vp);
    return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

}  // namespace

extern "C" {

const char *va_status_str(va_status s)
{
    switch (s) {
    case VA_OK: return "ok";
    case VA_ERR_INVALID_ARG: return "invalid argument";
    case VA_ERR_UNSUPPORTED: return "unsupported problem (outside the supported domain)";
    case VA_ERR_WORKSPACE: return "workspace missing or too small";
    case VA_ERR_HIP: return "HIP runtime error";
    case VA_ERR_DEVICE_DATA: return "invalid device metadata (validate mode)";
    }
    return "unknown status";
}

va_status va_plan(const va_problem *pr, va_plan_t *out)
{
    if (!pr || !out)
        return VA_ERR_INVALID_ARG;
    *out = nullptr;
    const va_problem &p = *pr;
    if (p.num_seqs < 1 || p.num_q_heads < 1 || p.num_kv_heads < 1 || p.head_dim < 1 ||
        p.page_size < 1 || p.max_seqlen_q < 1 || p.max_seqlen_k < 0 ||
        (p.layout == VA_LAYOUT_PAGED && p.max_blocks_per_seq < 1) ||
        p.num_blocks < 1 || p.total_q < 0 || p.num_cus < 0 || p.force_grid < 0 || p.force_grid > 65536)
        return VA_ERR_INVALID_ARG;
    if (p.total_q > (int64_t)p.num_seqs * p.max_seqlen_q)
        return VA_ERR_INVALID_ARG;
    if (p.q_dtype != VA_DT_BF16 && p.q_dtype != VA_DT_FP8_E4M3FN)
        return VA_ERR_INVALID_ARG;
    if (p.kv_dtype != VA_DT_BF16 && p.kv_dtype != VA_DT_FP8_E4M3FN)
        return VA_ERR_INVALID_ARG;
    if (p.q_dtype != VA_DT_BF16)
        return VA_ERR_UNSUPPORTED;
    if (p.layout != VA_LAYOUT_PAGED && p.layout != VA_LAYOUT_PREFIX_EXTEND)
        return VA_ERR_INVALID_ARG;
    const bool tok = p.layout == VA_LAYOUT_PREFIX_EXTEND;
    const int dv = p.v_head_dim == 0 ? p.head_dim : p.v_head_dim;
    if (p.v_head_dim < 0)
        return VA_ERR_INVALID_ARG;
    const bool mla = p.head_dim == kMlaDim;
    if (mla) {                                         // absorbed MLA: one kv head, paged, causal only
        if (dv != kMlaDv || p.num_kv_heads != 1 || tok || p.page_size != kPage || p.window_left != -1 ||
            p.softcap != 0.f)
            return VA_ERR_UNSUPPORTED;
    } else if (p.head_dim != kHeadDim || dv != kHeadDim || (!tok && p.page_size != kPage)) {
        return VA_ERR_UNSUPPORTED;
    }
    if (tok && p.num_blocks * (int64_t)p.page_size > INT32_MAX)    // buffer rows are int32 slots
        return VA_ERR_UNSUPPORTED;
    if (p.num_q_heads % p.num_kv_heads != 0)
        return VA_ERR_UNSUPPORTED;
    const int G = p.num_q_heads / p.num_kv_heads;
    if (G != 4 && G != 8 && G != 16)
        return VA_ERR_UNSUPPORTED;
    if (p.max_seqlen_q > 4)
        return VA_ERR_UNSUPPORTED;
    if (p.window_left < -1 || !(p.softcap >= 0.f) || p.softcap > 3.0e38f)
        return VA_ERR_INVALID_ARG;
    const bool fp8_paged = p.kv_dtype == VA_DT_FP8_E4M3FN && !tok && !mla;
    if (p.kernel < 0 || p.kernel > 2 || (p.kernel != 0 && !fp8_paged))
        return VA_ERR_INVALID_ARG;
    if (p.total_q * (int64_t)p.num_q_heads >= INT32_MAX)    // q rows are indexed with 32-bit integers
        return VA_ERR_UNSUPPORTED;
    const int64_t bh = (int64_t)p.num_seqs * p.num_kv_heads;
    const int64_t mbps = tok ? std::max<int64_t>(1, ((int64_t)p.max_seqlen_k + kPage - 1) / kPage)
                             : p.max_blocks_per_seq;
    if (bh > 65536 || bh * mbps > INT32_MAX)
        return VA_ERR_UNSUPPORTED;
    if (!tok && (int64_t)p.max_seqlen_k > (int64_t)p.max_blocks_per_seq * kPage)
        return VA_ERR_INVALID_ARG;

    int cus = p.num_cus;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return VA_ERR_HIP;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return VA_ERR_HIP;
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return VA_ERR_UNSUPPORTED;
        cus = prop.multiProcessorCount;
        if (cus < 1)
            return VA_ERR_HIP;
    }

    va_plan_s *pl = new (std::nothrow) va_plan_s;
    if (!pl)
        return VA_ERR_INVALID_ARG;
    pl->prob = p;
    pl->mbps = (int32_t)mbps;
    pl->log2g = G == 4 ? 2 : G == 8 ? 3 : 4;
    const int rows = G * p.max_seqlen_q;
    pl->rt = (rows + 15) / 16;
    pl->mla = mla;
    pl->rows_max = mla ? kMlaRows : 16 * 2 * (pl->rt <= 2 ? 1 : 2);   // 2 row groups x RTW row tiles
    pl->grid = p.force_grid > 0 ? p.force_grid : cus;
    // FP8 paged GQA: the one-wave-per-SIMD kernel streams a page faster, the
    // two-row-group kernel has about 6 us less fixed cost per piece (prologue
    // and epilogue).  Measured crossover at 96-128 pages per workgroup (long
    // context, 128: the first; 16 x 24576-key windows, 96: the second).
    {
        const int64_t keys = p.window_left >= 0
                                 ? std::min<int64_t>(p.max_seqlen_k, (int64_t)p.window_left + p.max_seqlen_q + kPage)
                                 : p.max_seqlen_k;
        const int64_t pages = bh * ((keys + kPage - 1) / kPage);
        pl->fp8_w4 = fp8_paged && (p.kernel == 1 || (p.kernel == 0 && pages >= 112 * (int64_t)pl->grid));
    }
    pl->min_pages = 8;
    pl->slots = 2 * (int64_t)pl->grid;                 // a first and a last piece per workgroup
    // Pages charged for a pair that starts inside a workgroup's share (see
    // locate): about the time of one more epilogue and prologue, in pages of
    // the kernel's own streaming rate (measured on the high-concurrency
    // workload for the FP8 cache; scaled by page bytes for the others).
    pl->piece_cost = mla ? (p.kv_dtype == VA_DT_FP8_E4M3FN ? 24 : 12)
                         : (p.kv_dtype == VA_DT_FP8_E4M3FN ? 32 : 16);
    if ((int64_t)bh * (mbps + pl->piece_cost) > INT32_MAX)
        pl->piece_cost = 0;                            // costs must stay 32-bit: split by pages
    size_t off = 256;                                   // meta
    pl->off_prefix = off;
    off = align_up(off + (size_t)(bh + 1) * 4, 256);
    pl->off_cost = off;
    off = align_up(off + (size_t)(bh + 1) * 4, 256);
    pl->off_lse = off;
    off = align_up(off + (size_t)pl->slots * pl->rows_max * 4, 256);
    pl->off_o = off;
    const size_t part_elt = p.kv_dtype == VA_DT_FP8_E4M3FN ? 2 : 4;   // fp16 or fp32 partial O
    off = align_up(off + (size_t)pl->slots * pl->rows_max * (mla ? kMlaDv : kHeadDim) * part_elt, 256);

    pl->ws_bytes = off;
    pl->debug = debug_env();
    if (pl->debug)
        fprintf(stderr,
                "va_plan: B=%d Hq=%d Hkv=%d G=%d max_q=%d max_k=%d mbps=%d blocks=%lld total_q=%lld "
                "kv=%s window_left=%d softcap=%g -> row_tiles=%d grid=%d min_pages=%d rows_max=%d "
                "slots=%lld workspace=%zu bytes (prefix @%zu, lse @%zu, partial O @%zu)\n",
                p.num_seqs, p.num_q_heads, p.num_kv_heads, G, p.max_seqlen_q, p.max_seqlen_k,
                p.max_blocks_per_seq, (long long)p.num_blocks, (long long)p.total_q,
                p.kv_dtype == VA_DT_FP8_E4M3FN ? "fp8" : "bf16", p.window_left, (double)p.softcap, pl->rt,
                pl->grid, pl->min_pages, pl->rows_max, (long long)pl->slots, pl->ws_bytes, pl->off_prefix,
                pl->off_lse, pl->off_o);
    *out = pl;
    return VA_OK;
}

va_status va_plan_workspace_bytes(va_plan_t plan, size_t *bytes)
{
    if (!plan || !bytes)
        return VA_ERR_INVALID_ARG;
    *bytes = plan->ws_bytes;
    return VA_OK;
}

va_status va_plan_kernel(va_plan_t plan, int32_t *kernel)
{
    if (!plan || !kernel)
        return VA_ERR_INVALID_ARG;
    const bool fp8_paged = plan->prob.kv_dtype == VA_DT_FP8_E4M3FN && plan->prob.layout == VA_LAYOUT_PAGED &&
                           !plan->mla;
    *kernel = !fp8_paged ? 0 : (plan->fp8_w4 ? 1 : 2);
    return VA_OK;
}

va_status va_plan_grid(va_plan_t plan, int32_t *grid)
{
    if (!plan || !grid)
        return VA_ERR_INVALID_ARG;
    *grid = plan->grid;
    return VA_OK;
}

void va_plan_destroy(va_plan_t plan)
{
    delete plan;
}

}  // extern "C"

namespace {

struct TokArgs {                 // prefix + extend layout arguments
    const int32_t *kv_indptr;
    const int32_t *kv_indices;
    int64_t num_kv_indices;
    const void *k_extend;
    const void *v_extend;
};

unsigned long long *g_stamps = nullptr;       // va_set_stamp_buffer (VA_STAMPS builds)
size_t g_stamp_bytes = 0;

va_status run_impl(va_plan_t plan, int32_t stage, const void *q, const void *k_pool, const void *v_pool,
                   const int32_t *block_table, const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                   const TokArgs *tok, float softmax_scale, const float *k_descale, const float *v_descale,
                   const float *sinks, void *out, void *workspace, size_t workspace_bytes, void *stream,
                   hipEvent_t main_start = nullptr, hipEvent_t main_stop = nullptr)
{
    if (!plan)
        return VA_ERR_INVALID_ARG;
    if (stage != VA_STAGE_ALL && stage != VA_STAGE_SPLIT_KV && stage != VA_STAGE_MERGE)
        return VA_ERR_INVALID_ARG;
    if ((tok != nullptr) != (plan->prob.layout == VA_LAYOUT_PREFIX_EXTEND))
        return VA_ERR_INVALID_ARG;                     // the entry point must match the plan's layout
    if (!q || !k_pool || !v_pool || !cu_seqlens_q || !out)
        return VA_ERR_INVALID_ARG;
    if (!tok && (!block_table || !seqused_k))
        return VA_ERR_INVALID_ARG;
    if (plan->mla && (k_pool != v_pool || sinks))      // V is the latent part of the K rows
        return VA_ERR_INVALID_ARG;
    if (tok) {
        if (!tok->kv_indptr || !tok->k_extend || !tok->v_extend || tok->num_kv_indices < 0 ||
            tok->num_kv_indices > INT32_MAX - 16 || (tok->num_kv_indices > 0 && !tok->kv_indices))
            return VA_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(tok->k_extend) | reinterpret_cast<uintptr_t>(tok->v_extend)) & 15)
            return VA_ERR_INVALID_ARG;
    }
    if (!workspace || workspace_bytes < plan->ws_bytes)
        return VA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return VA_ERR_INVALID_ARG;
    const uintptr_t align16 = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
                              reinterpret_cast<uintptr_t>(v_pool) | reinterpret_cast<uintptr_t>(out);
    if (align16 & 15)
        return VA_ERR_INVALID_ARG;
    const va_problem &pr = plan->prob;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);

    if (plan->debug && !tok && (stage == VA_STAGE_ALL || stage == VA_STAGE_SPLIT_KV)) {
        // validate mode: check the metadata first (result in workspace meta
        // words 2 and 3, which the kernels leave alone) and wait for it
        int32_t *res = reinterpret_cast<int32_t *>(ws) + 2;
        const va_status vs = enqueue_validate(plan, block_table, cu_seqlens_q, seqused_k, res, s);
        if (vs != VA_OK)
            return vs;
        int32_t h[2] = {0, 0};
        if (hipMemcpyAsync(h, res, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return VA_ERR_HIP;
        if (h[0] != 0) {
            fprintf(stderr, "va_run: invalid device metadata, bits 0x%x (1 cu_seqlens_q, 2 q_len > max_seqlen_q, "
                            "4 seqused_k, 8 q_len > seqused_k, 16 page id), first at sequence %d\n",
                    (unsigned)h[0], h[1]);
            return VA_ERR_DEVICE_DATA;
        }
    }

    if (stage == VA_STAGE_ALL || stage == VA_STAGE_SPLIT_KV) {
        SplitParams sp;
        sp.q = static_cast<const uint16_t *>(q);
        sp.k = static_cast<const uint8_t *>(k_pool);
        sp.v = static_cast<const uint8_t *>(v_pool);
        sp.bt = block_table;
        sp.cu = cu_seqlens_q;
        sp.seqused = seqused_k;
        sp.kdesc = k_descale;
        sp.vdesc = v_descale;
        sp.out = static_cast<uint16_t *>(out);
        sp.ws_o = ws + plan->off_o;
        sp.ws_lse = reinterpret_cast<float *>(ws + plan->off_lse);
        sp.ws_prefix = reinterpret_cast<int32_t *>(ws + plan->off_prefix);
        sp.ws_cost = reinterpret_cast<int32_t *>(ws + plan->off_cost);
        sp.ws_meta = reinterpret_cast<int32_t *>(ws);
        sp.piece_cost = plan->piece_cost;
        sp.scale_log2 = softmax_scale * 1.4426950408889634f;
        sp.cap_log2 = pr.softcap * 1.4426950408889634f;
        sp.sinks = sinks;
        sp.window_left = pr.window_left;
        sp.num_seqs = pr.num_seqs;
        sp.hq = pr.num_q_heads;
        sp.hkv = pr.num_kv_heads;
        sp.log2g = plan->log2g;
        sp.mbps = plan->mbps;
        sp.grid_n = plan->grid;
        sp.min_pages = plan->min_pages;
        sp.rows_max = plan->rows_max;
        sp.total_q = (int32_t)pr.total_q;
        sp.max_q = pr.max_seqlen_q;
        sp.num_blocks = pr.num_blocks;
        sp.kv_indptr = tok ? tok->kv_indptr : nullptr;
        sp.kv_indices = tok ? tok->kv_indices : nullptr;
        sp.kext = tok ? static_cast<const uint8_t *>(tok->k_extend) : nullptr;
        sp.vext = tok ? static_cast<const uint8_t *>(tok->v_extend) : nullptr;
        sp.num_indices = tok ? tok->num_kv_indices : 0;
        sp.num_rows = pr.num_blocks * pr.page_size;
        sp.stamps = g_stamp_bytes >= (size_t)plan->grid * 4 * kStampSlots * sizeof(unsigned long long) ? g_stamps
                                                                                                 : nullptr;
        const SplitKernel k = select_kernel(plan->rt, pr.kv_dtype == VA_DT_FP8_E4M3FN, pr.softcap > 0.f,
                                            tok != nullptr, plan->mla, plan->fp8_w4);
        void *args[] = {&sp};
        if (hipExtLaunchKernel(k.fn, dim3(plan->grid), dim3(k.threads), args, 0, s, main_start, main_stop, 0) !=
                hipSuccess ||
            hipGetLastError() != hipSuccess)
            return VA_ERR_HIP;
    }
    if (stage == VA_STAGE_ALL || stage == VA_STAGE_MERGE) {
        MergeParams mp;
        mp.cu = cu_seqlens_q;
        mp.vdesc = v_descale;
        mp.sinks = sinks;
        mp.ws_o = ws + plan->off_o;
        mp.ws_lse = reinterpret_cast<const float *>(ws + plan->off_lse);
        mp.ws_prefix = reinterpret_cast<const int32_t *>(ws + plan->off_prefix);
        mp.ws_cost = reinterpret_cast<const int32_t *>(ws + plan->off_cost);
        mp.ws_meta = reinterpret_cast<const int32_t *>(ws);
        mp.out = static_cast<uint16_t *>(out);
        mp.num_seqs = pr.num_seqs;
        mp.hq = pr.num_q_heads;
        mp.hkv = pr.num_kv_heads;
        mp.log2g = plan->log2g;
        mp.max_q = pr.max_seqlen_q;
        mp.rows_max = plan->rows_max;
        mp.total_q = (int32_t)pr.total_q;
        const int hpb = plan->mla ? 2 : 1;                 // heads per merge workgroup
        const int64_t blocks = (int64_t)pr.num_seqs * pr.num_kv_heads * pr.max_seqlen_q *
                               ((pr.num_q_heads / pr.num_kv_heads) / hpb);
        if (blocks > 0) {
            const bool half = pr.kv_dtype == VA_DT_FP8_E4M3FN;
            void (*merge)(MergeParams) =
                plan->mla ? (half ? va_merge_kernel<true, kMlaDv, kThreads> : va_merge_kernel<false, kMlaDv, kThreads>)
                          : (half ? va_merge_kernel<true, kHeadDim, kMergeThreadsGqa>
                                  : va_merge_kernel<false, kHeadDim, kMergeThreadsGqa>);
            hipLaunchKernelGGL(merge, dim3((unsigned)blocks), dim3(plan->mla ? kThreads : kMergeThreadsGqa), 0, s, mp);
            if (hipGetLastError() != hipSuccess)
                return VA_ERR_HIP;
        }
    }
    return VA_OK;
}

// ------------------------------------------------ no-allocation entry point --
//
// va_run_noalloc runs the same kernels with a workspace that lives in this
// library's own device memory: the file-scope array `scratch` (each device
// that loads the library holds one copy until the process ends).  In host code
// the name `scratch` is only a stand-in for the symbol, so the array's device
// address is looked up once per device with hipGetSymbolAddress and kept; only
// that address is ever passed to a kernel.  The kernels need no zeroed
// workspace: every word they read in it was written earlier in the same call.
constexpr size_t kScratchBytes = (size_t)80 << 20;
__device__ __align__(256) static unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

va_status scratch_address(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return VA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return VA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return VA_OK;
}

}  // namespace

extern "C" {

va_status va_run_ex(va_plan_t plan, int32_t stage, const void *q, const void *k_pool,
                    const void *v_pool, const int32_t *block_table,
                    const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                    float softmax_scale, const float *k_descale, const float *v_descale,
                    const float *sinks, void *out, void *workspace, size_t workspace_bytes,
                    void *stream)
{
    return run_impl(plan, stage, q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, nullptr,
                    softmax_scale, k_descale, v_descale, sinks, out, workspace, workspace_bytes, stream);
}

va_status va_run_prefix_extend(va_plan_t plan, int32_t stage, const void *q, const void *k_buffer,
                               const void *v_buffer, const int32_t *kv_indptr, const int32_t *kv_indices,
                               int64_t num_kv_indices, const void *k_extend, const void *v_extend,
                               const int32_t *cu_seqlens_q, float softmax_scale, const float *k_descale,
                               const float *v_descale, const float *sinks, void *out, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    const TokArgs tok = {kv_indptr, kv_indices, num_kv_indices, k_extend, v_extend};
    return run_impl(plan, stage, q, k_buffer, v_buffer, nullptr, cu_seqlens_q, nullptr, &tok, softmax_scale,
                    k_descale, v_descale, sinks, out, workspace, workspace_bytes, stream);
}

va_status va_run_timed(va_plan_t plan, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_table, const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                       float softmax_scale, const float *k_descale, const float *v_descale, const float *sinks,
                       void *out, void *workspace, size_t workspace_bytes, void *stream, void *main_start,
                       void *main_stop)
{
    if (!main_start || !main_stop)
        return VA_ERR_INVALID_ARG;
    return run_impl(plan, VA_STAGE_ALL, q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, nullptr,
                    softmax_scale, k_descale, v_descale, sinks, out, workspace, workspace_bytes, stream,
                    reinterpret_cast<hipEvent_t>(main_start), reinterpret_cast<hipEvent_t>(main_stop));
}

va_status va_set_stamp_buffer(void *buffer, size_t bytes)
{
#ifdef VA_STAMPS
    g_stamps = static_cast<unsigned long long *>(buffer);
    g_stamp_bytes = buffer ? bytes : 0;
    return VA_OK;
#else
    (void)buffer;
    (void)bytes;
    return VA_ERR_UNSUPPORTED;
#endif
}

va_status va_run(va_plan_t plan, const void *q, const void *k_pool, const void *v_pool,
                 const int32_t *block_table, const int32_t *cu_seqlens_q,
                 const int32_t *seqused_k, float softmax_scale, const float *k_descale,
                 const float *v_descale, void *out, void *workspace, size_t workspace_bytes,
                 void *stream)
{
    return va_run_ex(plan, VA_STAGE_ALL, q, k_pool, v_pool, block_table, cu_seqlens_q,
                     seqused_k, softmax_scale, k_descale, v_descale, nullptr, out, workspace,
                     workspace_bytes, stream);
}

va_status va_run_noalloc(va_plan_t plan, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *block_table, const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                         float softmax_scale, const float *k_descale, const float *v_descale,
                         const float *sinks, void *out, void *stream)
{
    if (!plan)
        return VA_ERR_INVALID_ARG;
    if (plan->ws_bytes > kScratchBytes)
        return VA_ERR_WORKSPACE;                       // beyond the library's scratch
    void *ws = nullptr;
    const va_status st = scratch_address(&ws);
    if (st != VA_OK)
        return st;
    return run_impl(plan, VA_STAGE_ALL, q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, nullptr,
                    softmax_scale, k_descale, v_descale, sinks, out, ws, kScratchBytes, stream);
}

va_status va_validate(va_plan_t plan, const int32_t *block_table, const int32_t *cu_seqlens_q,
                      const int32_t *seqused_k, int32_t *result, void *stream)
{
    if (!plan || !block_table || !cu_seqlens_q || !seqused_k || !result)
        return VA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(result) & 3)
        return VA_ERR_INVALID_ARG;
    return enqueue_validate(plan, block_table, cu_seqlens_q, seqused_k, result,
                            reinterpret_cast<hipStream_t>(stream));
}

va_status va_spec_block_table(const int32_t *kv_indptr, const int32_t *kv_indices, int32_t num_seqs,
                              int32_t page_size, int32_t max_blocks_per_seq, int32_t *block_table,
                              int32_t *seqused_k, void *stream)
{
    if (!kv_indptr || !kv_indices || !block_table || !seqused_k || num_seqs < 1 || page_size < 1 ||
        max_blocks_per_seq < 1)
        return VA_ERR_INVALID_ARG;
    const int64_t n = (int64_t)num_seqs * max_blocks_per_seq;
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > INT32_MAX)
        return VA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(va_spec_block_table_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), kv_indptr, kv_indices, num_seqs, page_size,
                       max_blocks_per_seq, block_table, seqused_k);
    return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

va_status va_stream_pages(const void *pool, int64_t pool_bytes, const int32_t *pages, int64_t npages,
                          int32_t depth, int32_t grid, uint32_t *sums, void *stream)
{
    if (!pool || !pages || !sums || npages < 0 || pool_bytes < 4096 || grid < 1 || grid > 65536 ||
        (reinterpret_cast<uintptr_t>(pool) & 15) != 0)
        return VA_ERR_INVALID_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void (*k)(const uint8_t *, int64_t, const int32_t *, int64_t, uint32_t *) = nullptr;
    switch (depth) {
    case 2: k = va_stream_pages_kernel<2>; break;
    case 4: k = va_stream_pages_kernel<4>; break;
    case 6: k = va_stream_pages_kernel<6>; break;
    case 8: k = va_stream_pages_kernel<8>; break;
    case 10: k = va_stream_pages_kernel<10>; break;
    default: return VA_ERR_INVALID_ARG;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint8_t *>(pool),
                       pool_bytes / 4096, pages, npages, sums);
    return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

va_status va_fp8_to_bf16(const uint8_t *in, uint16_t *out, int64_t n, void *stream)
{
    if (n < 0 || (n > 0 && (!in || !out)))
        return VA_ERR_INVALID_ARG;
    if (n == 0)
        return VA_OK;
    const int64_t threads = (n + 3) / 4;
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(va_fp8_to_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), in, out, n);
    return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

}  // extern "C"
