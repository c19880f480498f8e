// k_attn.hip -- gathered gated GQA attention over the selected blocks (gfx950).
//
// ai.info "StepFun Details Step 5 Preview's 92-Block Agent Design", section
// "Why StepFun chose 92 transformer blocks": the full-attention layers are
// Gated Grouped-Query Attention; section "Sparse GQA targets million-token
// context": they attend only to the selected historical blocks.  ai4snews
// Interpretation para. 2 names a sparse flash-attention operator for this.
//
// One wave owns one (query token, KV group): the 16 query heads of the group
// are the M dimension of v_mfma_f32_16x16x32_bf16, so every gathered K/V row
// feeds 16 heads.  Per step of 32 token slots (4 blocks of 8):
//   S^T[slot][head] = K_rows . Q^T   (K rows loaded straight into the A operand)
//   online softmax in fp32, base-2 domain, per head (= lane % 16)
//   O^T[d][head]   += V^T . P^T      (V rows staged in LDS, read transposed)
// The P^T operand is exactly the layout S^T leaves in the registers once the
// contraction slots are ordered {4q..4q+3, 16+4q..16+4q+3} for lane row q,
// so no register shuffle is needed between the two products.
// Prefill: one workgroup per query token, one wave per KV group (the rows of
// all groups of a token are adjacent in memory).  Decode: the selected blocks
// of each (sequence, group) are split across workgroups and the partial
// softmax states are merged exactly afterwards.
#include <hip/hip_runtime.h>

#include "sgqa_device.hpp"
#include "sgqa_launch.hpp"

namespace sgqa {

constexpr int kSlots = 32;  // token slots per step

// Each wave stages V in its own LDS region, so only the wave's own LDS operations need
// ordering: they execute in issue order, and these fences keep the compiler from moving
// LDS accesses across the hand-off.  Waves of one workgroup never wait for each other.
// This thread's wave within the workgroup, as a wave-uniform (scalar) value: values derived
// from it (rows, groups, pointers) then live in scalar registers.
__device__ __forceinline__ int wave_index()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}


// Column reads of a [row][d] bf16 tile in LDS (row stride ld elements, a multiple of 4) by the
// transposing read ds_read_b64_tr_b16 (gfx950).  Within each 16-lane group, lane i receives
// element i % 4 of the 8-byte chunks read by lanes i / 4 + {0, 4, 8, 12}; so when lane L reads
// row 4 q4 + L / 4, columns d0 + 4 (L % 4) .. +3, lane (col, q4) receives
// tile[4 q4 + j][d0 + col] for j = 0..3: one 16x16x16 MFMA operand quad.
typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 tr_quad(const uint16_t *tile, int ld, int d0)
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const uint16_t *p = tile + (q4 * 4 + (col >> 2)) * ld + d0 + 4 * (col & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)p);
}

// The MFMA A operand V^T[d0 + col][slots] of a [slot][d] tile: the slots {4 q4 .. 4 q4 + 3}
// then {16 + 4 q4 .. 16 + 4 q4 + 3}, the contraction order P^T uses.
__device__ __forceinline__ bf16x8 vt_fragment(const uint16_t *tile, int ld, int d0)
{
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = __builtin_shufflevector(tr_quad(tile, ld, d0), tr_quad(tile + 16 * ld, ld, d0),
                                            0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

template <int D>
struct WaveState {
    f32x4 acc[D / 16];  // acc[mt][i] = O^T[d = 16*mt + 4*q + i][head = lane % 16]
    float m;            // running max of the base-2 logits of this lane's head
    float l;            // this lane's share of the denominator, summing the bf16 weights PV uses
    float l32;          // the same share summing the fp32 weights (for the log-sum-exp)
};

// Where the tokens of one query come from, 32 slots per step.
// SparseTokens: the selected blocks idx[e_begin, e_end) of a query at t (own block c);
// slots beyond t, -1 entries and ids outside [0, c] are invalid.
// Selection entries a wave keeps in its LDS window.
constexpr int kWin = 256;

// The tokens a wave attends: the selected blocks sel[e_begin, e_end) of query position t (own
// block c), kSlots tokens per step.  Each step's entries come from the wave's LDS window `win`,
// refilled by one coalesced read of the next kWin entries only when a step runs past it, so the
// gathers of a step never wait on a global load of its entries.
struct SparseTokens {
    const int32_t *sel;
    int e_begin, e_end;
    int64_t t, c;
    int B;
    int32_t *win;
    __device__ int steps() const
    {
        const int eps = kSlots / B;
        return (e_end - e_begin + eps - 1) / eps;
    }
    // Block of slot sl at step `step` (-1 past e_end); wbase = first entry in the window
    // (start it below any entry, e.g. INT_MIN / 2).  Uniform across the wave except for sl.
    __device__ int32_t block(int step, int sl, int &wbase) const
    {
        const int e0 = e_begin + step * (kSlots / B);
        if (e0 + kSlots / B > wbase + kWin) {
            const int lane = threadIdx.x & 63;
            int32_t v[kWin / 64];
#pragma unroll
            for (int j = 0; j < kWin / 64; ++j) {  // in-range reads, issued together
                const int e = e0 + lane + 64 * j;
                v[j] = sel[e < e_end ? e : e_end - 1];
                v[j] = e < e_end ? v[j] : -1;
            }
            wave_lds_handoff();
#pragma unroll
            for (int j = 0; j < kWin / 64; ++j)
                win[lane + 64 * j] = v[j];
            wave_lds_handoff();
            wbase = e0;
        }
        return win[e0 - wbase + sl / B];
    }
    // Token of slot sl: clamped load position + validity.
    __device__ void slot(int step, int sl, int &wbase, int64_t &s_ld, bool &valid) const
    {
        const int32_t blk = block(step, sl, wbase);
        const int64_t s = (int64_t)blk * B + (sl % B);
        valid = blk >= 0 && (int64_t)blk <= c && s <= t;
        s_ld = valid ? s : t;
    }
};

// A wave's V (or K) staging buffer of the sparse kernels: kSlots rows of D + 8 bf16 (elements).
constexpr int attn_vbuf_elems(int D)
{
    return kSlots * (D + 8);
}

// LDS bytes per wave of the sparse kernels: V buffer plus the entry window.
constexpr size_t attn_wave_lds(int D)
{
    return (size_t)attn_vbuf_elems(D) * sizeof(uint16_t) + kWin * sizeof(int32_t);
}

// This wave's entry window: after the workgroup's V buffers.
template <int D>
__device__ __forceinline__ int32_t *entry_window(uint16_t *lds)
{
    const int nw = blockDim.x >> 6, wave = wave_index();
    return reinterpret_cast<int32_t *>(lds + nw * attn_vbuf_elems(D)) + wave * kWin;
}

// Where the K/V rows of one KV group g come from.  Bf16Rows: Kg/Vg point at element
// (token 0, group g, dim 0) of a bf16 cache; rows are Hkv*D elements apart.
struct Bf16Rows {
    static constexpr bool kFp8 = false;
    static constexpr bool kStream = false;
    const uint16_t *Kg, *Vg;
};
// Rows the kernel reads once (the decode's gathers): non-temporal loads, 49.5 -> 45.0 us for
// the decode attention of 16 x 1M (the FP8 rows measured slower that way)
struct Bf16StreamRows : Bf16Rows {
    static constexpr bool kStream = true;
};
// Fp8Rows: e4m3 codes laid out the same way (one byte per element), and one fp32 scale per
// (token, group) at Ks[token * Hkv] / Vs[token * Hkv]: the row's values are code * scale.
struct Fp8Rows {
    static constexpr bool kFp8 = true;
    static constexpr bool kStream = false;
    const uint8_t *Kg, *Vg;
    const float *Ks, *Vs;
};

template <typename Rows>
__device__ __forceinline__ u32x4 load_row(const void *p)
{
    if constexpr (Rows::kStream)
        return load16_stream(p);
    else
        return load16(p);
}

// Online softmax with a lazy running maximum: a step moves a query's (or head's) maximum only
// when it raises it by more than kLazyMax in log2 units, so most steps keep the maximum and
// skip the rescale of the accumulators; the weights exp2(x - m) then stay below 2^kLazyMax,
// well inside the range of fp32 sums and bf16 weights, and the output and lse use the same m
// as the sums.
#ifndef SGQA_LAZY_MAX
#define SGQA_LAZY_MAX 8.0f
#endif
constexpr float kLazyMax = SGQA_LAZY_MAX;

// The query operand of Sᵀ = K·Qᵀ: fragment kk holds dims [32 kk + 8 q4, +8) of head col
// (lane = 16 q4 + col), in registers (load_q / load_q_perm).
template <int D>
struct QRegs {
    const bf16x8 (&f)[D / 32];
    __device__ __forceinline__ bf16x8 operator()(int kk) const { return f[kk]; }
};

// One 32-slot step's rows of a wave, as loaded into registers: for bf16 rows, the K and V
// pieces of whole rows (flat piece f = lane + 64 ci covers slot f / pieces, piece f % pieces:
// pieces of 8 values, or of 16 FP8 codes, so each load instruction reads whole rows); for FP8
// rows, the K codes straight in the A-operand layout and the row scales of this lane's slot
// (lane & 31).
template <int D, bool kFp8>
struct StepRows {
    static constexpr int kVPieces = kFp8 ? D / 16 : D / 8;
    static constexpr int kVLoads = kFp8 ? D / 32 : D / 16;
    static constexpr int kKLoads = kFp8 ? D / 64 : 1;
    u32x4 kv[2][kKLoads];
    u32x4 kp[kFp8 ? 1 : kVLoads];
    u32x4 vv[kVLoads];
    float k_scale, v_scale;
};

// The tokens of one step: slot validity (bit per slot) and this lane's slot (lane & 31)
// clamped load position, split in 32-bit halves for the shuffles.
struct StepSlots {
    uint64_t vmask;
    int64_t s_ld;
    int s_lo, s_hi;
};

// Reads the wave's entry window, which it refills from the selection row when the step runs
// past it.
template <typename Src>
__device__ __forceinline__ StepSlots step_slots(const Src &src, int step, int &wbase)
{
    StepSlots p;
    bool valid;
    src.slot(step, (int)(threadIdx.x & 31), wbase, p.s_ld, valid);
    p.vmask = __ballot(valid);
    p.s_lo = (int)(p.s_ld & 0xffffffff);
    p.s_hi = (int)(p.s_ld >> 32);
    return p;
}

// Address of element `elem` of the row of slot `slot` (the token p.s_ld of lane `slot`).
template <typename T>
__device__ __forceinline__ const T *row_piece(const T *base, const StepSlots &p, int slot,
                                              int64_t row_elems, int elem)
{
    const int64_t sv = ((int64_t)(uint32_t)__shfl(p.s_lo, slot)) |
                       ((int64_t)__shfl(p.s_hi, slot) << 32);
    return base + sv * row_elems + elem;
}

// Issue the K loads of a step.  bf16 K rows are read whole and staged in LDS for the A
// operands: read straight in the operand layout (16 rows x 64 bytes per instruction) the same
// gathers took 135 instead of 113 ms in a loads-only copy of the 128K prefill.
template <int D, typename Rows>
__device__ __forceinline__ void issue_k(const Rows &rows, int Hkv, const StepSlots &p,
                                        StepRows<D, Rows::kFp8> &r)
{
    using SR = StepRows<D, Rows::kFp8>;
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const int64_t row_elems = (int64_t)Hkv * D;
    if constexpr (Rows::kFp8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int src_lane = h * 16 + col;
            const int64_t sk = ((int64_t)(uint32_t)__shfl(p.s_lo, src_lane)) |
                               ((int64_t)__shfl(p.s_hi, src_lane) << 32);
            const uint8_t *kr = rows.Kg + sk * row_elems + q4 * 16;
#pragma unroll
            for (int k2 = 0; k2 < SR::kKLoads; ++k2)
                r.kv[h][k2] = load16(kr + k2 * 64);
        }
    } else {
#pragma unroll
        for (int ci = 0; ci < SR::kVLoads; ++ci) {
            const int f = lane + 64 * ci;
            const int slot = f / SR::kVPieces, piece = f - slot * SR::kVPieces;
            r.kp[ci] = load16(row_piece(rows.Kg, p, slot, row_elems, piece * 8));
        }
    }
}

// Issue the V loads of a step (and, for FP8 rows, the row scales of this lane's slot).
template <int D, typename Rows>
__device__ __forceinline__ void issue_v(const Rows &rows, int Hkv, const StepSlots &p,
                                        StepRows<D, Rows::kFp8> &r)
{
    using SR = StepRows<D, Rows::kFp8>;
    const int lane = threadIdx.x & 63;
    const int64_t row_elems = (int64_t)Hkv * D;
#pragma unroll
    for (int ci = 0; ci < SR::kVLoads; ++ci) {
        const int f = lane + 64 * ci;
        const int slot = f / SR::kVPieces, piece = f - slot * SR::kVPieces;
        if constexpr (Rows::kFp8)
            r.vv[ci] = load16(row_piece(rows.Vg, p, slot, row_elems, piece * 16));
        else
            r.vv[ci] = load16(row_piece(rows.Vg, p, slot, row_elems, piece * 8));
    }
    r.k_scale = 1.0f;
    r.v_scale = 1.0f;
    if constexpr (Rows::kFp8) {
        r.k_scale = rows.Ks[p.s_ld * Hkv];
        r.v_scale = rows.Vs[p.s_ld * Hkv];
    }
}

// Issue all loads of a step; bf16 K and V pieces of a row share one offset computation.
template <int D, typename Rows>
__device__ __forceinline__ void issue_kv(const Rows &rows, int Hkv, const StepSlots &p,
                                         StepRows<D, Rows::kFp8> &r)
{
    if constexpr (Rows::kFp8) {
        issue_k<D>(rows, Hkv, p, r);
        issue_v<D>(rows, Hkv, p, r);
    } else {
        using SR = StepRows<D, false>;
        const int lane = threadIdx.x & 63;
        const int64_t row_elems = (int64_t)Hkv * D;
#pragma unroll
        for (int ci = 0; ci < SR::kVLoads; ++ci) {
            const int f = lane + 64 * ci;
            const int slot = f / SR::kVPieces, piece = f - slot * SR::kVPieces;
            const int64_t sv = ((int64_t)(uint32_t)__shfl(p.s_lo, slot)) |
                               ((int64_t)__shfl(p.s_hi, slot) << 32);
            const int64_t off = sv * row_elems + piece * 8;
            r.kp[ci] = load_row<Rows>(rows.Kg + off);
            r.vv[ci] = load_row<Rows>(rows.Vg + off);
        }
        r.k_scale = 1.0f;
        r.v_scale = 1.0f;
    }
}

// Sᵀ = K·Qᵀ for slots 0-15 (sc[0]) and 16-31 (sc[1]).  bf16: the K rows are first staged in
// the wave's buffer `vs` [kSlots][D + 8] (the previous step's transposed V reads are done at
// the handoff) and the A operands read from it.  FP8: the query fragments must be in the
// permuted dim order of load_q_perm; each 16 codes feed two MFMA steps after an exact
// conversion to bf16, and the row's K scale multiplies its logits.
template <int D, bool kFp8, typename Q>
__device__ __forceinline__ void step_scores(const StepRows<D, kFp8> &r, const Q &qf, uint16_t *vs,
                                            f32x4 (&sc)[2])
{
    using SR = StepRows<D, kFp8>;
    constexpr int kLd = D + 8;  // LDS row stride in elements (conflict-free transposing reads)
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    if constexpr (!kFp8) {
        wave_lds_handoff();
#pragma unroll
        for (int ci = 0; ci < SR::kVLoads; ++ci) {
            const int f = lane + 64 * ci;
            const int slot = f / SR::kVPieces, piece = f - slot * SR::kVPieces;
            uint2 *dst = reinterpret_cast<uint2 *>(vs + slot * kLd + piece * 8);
            dst[0] = uint2{r.kp[ci][0], r.kp[ci][1]};
            dst[1] = uint2{r.kp[ci][2], r.kp[ci][3]};
        }
        wave_lds_handoff();
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        sc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kFp8) {
#pragma unroll
            for (int k2 = 0; k2 < SR::kKLoads; ++k2) {
                bf16x8 lo, hi;
                e4m3x16_to_bf16x8x2(r.kv[h][k2], lo, hi);
                sc[h] = mfma_16x16x32(lo, qf(2 * k2), sc[h]);
                sc[h] = mfma_16x16x32(hi, qf(2 * k2 + 1), sc[h]);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const u32x4 ka = *reinterpret_cast<const u32x4 *>(
                    vs + (h * 16 + col) * kLd + kk * 32 + q4 * 8);
                sc[h] = mfma_16x16x32(as_bf16x8(ka), qf(kk), sc[h]);
            }
        }
    }
}

// Online softmax (base 2) of one step's scores; returns the Pᵀ operand of the PV product.
// Lane holds slots 16h + 4*q4 + i of head col.  The weights are normalised by their bf16
// values, the ones PV uses, so the output is a convex combination; with FP8 rows each V
// row's scale rides on its weight.
template <int D, bool kFp8>
__device__ __forceinline__ bf16x8 step_softmax(const f32x4 (&sc_in)[2], uint64_t vmask,
                                               float k_scale, float v_scale, float scale_log2,
                                               WaveState<D> &st)
{
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const float neg_inf = -__builtin_inff();
    f32x4 sc[2] = {sc_in[0], sc_in[1]};
    if constexpr (kFp8) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[h][i] *= __shfl(k_scale, h * 16 + q4 * 4 + i);
    }
    float x[2][4];
    float mloc = neg_inf;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = h * 16 + q4 * 4 + i;
            const bool ok = (vmask >> slot) & 1ull;
            x[h][i] = ok ? sc[h][i] * scale_log2 : neg_inf;
            mloc = fmaxf(mloc, x[h][i]);
        }
    // the running maximum moves only when a step raises it by more than kLazyMax (log2
    // units), so most steps skip the accumulators' rescale (wave vote); the weights stay
    // below 2^kLazyMax
    const float m_row = fmaxf(st.m, max_across_rows(mloc));
    const float m_new = m_row > st.m + kLazyMax ? m_row : st.m;
    const bool any = m_new != neg_inf;
    const float alpha = any ? fast_exp2(st.m - m_new) : 1.0f;
    float p[2][4];
    float psum = 0.f, psum32 = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pe = any ? fast_exp2(x[h][i] - m_new) : 0.f;
            p[h][i] = bf16_bits_to_f32(f32_to_bf16_bits(pe));
            psum += p[h][i];
            psum32 += pe;
            if constexpr (kFp8)
                p[h][i] = pe * __shfl(v_scale, h * 16 + q4 * 4 + i);
        }
    st.l = st.l * alpha + psum;
    st.l32 = st.l32 * alpha + psum32;
    st.m = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st.acc[mt][i] *= alpha;
    }
    u32x4 pw;
    pw[0] = pack_bf16x2(p[0][0], p[0][1]);
    pw[1] = pack_bf16x2(p[0][2], p[0][3]);
    pw[2] = pack_bf16x2(p[1][0], p[1][1]);
    pw[3] = pack_bf16x2(p[1][2], p[1][3]);
    return as_bf16x8(pw);
}

// Stage a step's V rows in the wave's buffer (FP8 codes converted to bf16 on the way).
template <int D, bool kFp8>
__device__ __forceinline__ void stage_v(const StepRows<D, kFp8> &r, uint16_t *vs)
{
    using SR = StepRows<D, kFp8>;
    constexpr int kLd = D + 8;
    const int lane = threadIdx.x & 63;
    wave_lds_handoff();
#pragma unroll
    for (int ci = 0; ci < SR::kVLoads; ++ci) {
        const int f = lane + 64 * ci;
        const int slot = f / SR::kVPieces, piece = f - slot * SR::kVPieces;
        if constexpr (kFp8) {
            uint32_t w[8];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                e4m3x4_to_bf16(r.vv[ci][e], w[2 * e], w[2 * e + 1]);
            uint2 *dst = reinterpret_cast<uint2 *>(vs + slot * kLd + piece * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[e] = uint2{w[2 * e], w[2 * e + 1]};
        } else {
            uint2 *dst = reinterpret_cast<uint2 *>(vs + slot * kLd + piece * 8);
            dst[0] = uint2{r.vv[ci][0], r.vv[ci][1]};
            dst[1] = uint2{r.vv[ci][2], r.vv[ci][3]};
        }
    }
    wave_lds_handoff();
}

// Oᵀ += Vᵀ·Pᵀ from the staged V rows: A[m = d][k = slot perm(8*q4 + j)], slots 4q4+j (j<4),
// 16+4q4+j-4.
template <int D>
__device__ __forceinline__ void step_pv(const uint16_t *vs, bf16x8 pf, WaveState<D> &st)
{
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        st.acc[mt] = mfma_16x16x32(vt_fragment(vs, D + 8, mt * 16), pf, st.acc[mt]);
}

// Attend one wave's (token, group) over the tokens of `src`, reading rows from `rows`, one
// 32-slot step at a time (`vs`: the wave's LDS buffer [kSlots][D + 8]).  Per step the K rows
// feed Sᵀ = K·Qᵀ, an online softmax gives Pᵀ, and the V rows, staged in `vs` and read
// transposed, feed Oᵀ += Vᵀ·Pᵀ.
template <int D, typename Src, typename Rows, typename Q>
__device__ __forceinline__ void attend_range(const Rows &rows, int Hkv, const Src &src,
                                             const Q &qf, float scale_log2, uint16_t *vs,
                                             WaveState<D> &st)
{
    constexpr bool kFp8 = Rows::kFp8;
    const int nsteps = src.steps();
    int wbase = -(1 << 30);  // empty window
    for (int step = 0; step < nsteps; ++step) {
        const StepSlots p = step_slots(src, step, wbase);
        StepRows<D, kFp8> r;
        issue_kv<D>(rows, Hkv, p, r);
        f32x4 sc[2];
        step_scores<D, kFp8>(r, qf, vs, sc);
        const bf16x8 pf = step_softmax<D, kFp8>(sc, p.vmask, r.k_scale, r.v_scale, scale_log2,
                                                st);
        stage_v<D, kFp8>(r, vs);
        step_pv<D>(vs, pf, st);
    }
}

template <int D>
__device__ __forceinline__ void load_q(const uint16_t *__restrict__ qh, int hpg, bf16x8 (&qf)[D / 32])
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (col < hpg)
            v = load16(qh + (int64_t)col * D + kk * 32 + q4 * 8);
        qf[kk] = as_bf16x8(v);
    }
}

// Query fragments in the dim order the FP8 rows use: qf[2 k2 + h] holds dims
// [64 k2 + 16 q4 + 8 h, +8) of head col (D a multiple of 64).
template <int D>
__device__ __forceinline__ void load_q_perm(const uint16_t *__restrict__ qh, int hpg,
                                            bf16x8 (&qf)[D / 32])
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int k2 = 0; k2 < D / 64; ++k2) {
        u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
        if (col < hpg) {
            v0 = load16(qh + (int64_t)col * D + k2 * 64 + q4 * 16);
            v1 = load16(qh + (int64_t)col * D + k2 * 64 + q4 * 16 + 8);
        }
        qf[2 * k2] = as_bf16x8(v0);
        qf[2 * k2 + 1] = as_bf16x8(v1);
    }
}

template <int D>
__device__ __forceinline__ void init_state(WaveState<D> &st)
{
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        st.acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -__builtin_inff();
    st.l = 0.f;
    st.l32 = 0.f;
}

__device__ __forceinline__ float sigmoid_f32(float x)
{
    return 1.0f / (1.0f + fast_exp2(-x * 1.4426950408889634f));
}

// Normalise, gate and store one (row, group): out[r][g*hpg + head][:] and lse.
template <int D>
__device__ __forceinline__ void store_row(const WaveState<D> &st, const AttnArgs &a, int64_t r,
                                          int g, int hpg)
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const float l = sum_across_rows(st.l);
    const float l32 = sum_across_rows(st.l32);
    if (col < hpg) {
        const int h = g * hpg + col;
        const float gsig = sigmoid_f32(bf16_bits_to_f32(a.gate[r * a.Hq + h]));
        const float f = gsig / l;
        uint16_t *o = a.out + (r * a.Hq + h) * D + q4 * 4;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
            uint2 w;
            w.x = pack_bf16x2(st.acc[mt][0] * f, st.acc[mt][1] * f);
            w.y = pack_bf16x2(st.acc[mt][2] * f, st.acc[mt][3] * f);
            *reinterpret_cast<uint2 *>(o + mt * 16) = w;
        }
        if (a.lse && q4 == 0)
            a.lse[r * a.Hq + h] = (st.m + fast_log2(l32)) * 0.6931471805599453f;
    }
}

// Between the launches of a sliced prefill each wave parks its raw register state (the
// 4*(D/16) accumulator values, max and the two partial sums of every lane) in the
// workspace, in lane order, so the next launch resumes exactly where this one stopped.
template <int D>
constexpr int state_floats()
{
    return 4 * (D / 16) + 4;  // + m, l, l32, pad
}

__device__ __forceinline__ int64_t state_offset(const AttnArgs &a, int64_t r, int g)
{
    return ((r * a.Hkv + g) * 64) * (int64_t)a.state_stride + (threadIdx.x & 63) * a.state_stride;
}

template <int D>
__device__ __forceinline__ void save_state(const WaveState<D> &st, float *p)
{
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        *reinterpret_cast<f32x4 *>(p + 4 * mt) = st.acc[mt];
    *reinterpret_cast<f32x4 *>(p + 4 * (D / 16)) = f32x4{st.m, st.l, st.l32, 0.f};
}

template <int D>
__device__ __forceinline__ void load_state(WaveState<D> &st, const float *p)
{
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        st.acc[mt] = *reinterpret_cast<const f32x4 *>(p + 4 * mt);
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p + 4 * (D / 16));
    st.m = v[0];
    st.l = v[1];
    st.l32 = v[2];
}

// Histories of more than this many slice_blocks ranges are cut into long_slices ranges.
constexpr int64_t kMaxBaseSlices = 16;

// Row and group of this wave under the two workgroup mappings (see k_attn_prefill).
// Returns false for waves past the last row.
template <bool kGroupPerXcd, typename Args>
__device__ __forceinline__ bool wave_row_group(const Args &a, int64_t &r, int &g)
{
    const int wave = wave_index();
    if constexpr (kGroupPerXcd) {
        const int R = 8 / a.Hkv;
        const int x = blockIdx.x & 7;
        g = x / R;
        const int64_t tile = (int64_t)(blockIdx.x >> 3) * R + (x % R);
        const int64_t row = tile * 4 + wave;
        if (row >= a.rows)
            return false;
        r = (int64_t)a.rows - 1 - row;  // longest rows first
    } else {
        r = (int64_t)a.rows - 1 - blockIdx.x;
        g = wave;
    }
    return true;
}

// kGroupPerXcd: workgroups are dispatched round-robin over the 8 XCDs; XCD x serves KV
// group x / (8 / Hkv) only, so each XCD's L2 holds one group's K/V rows, and the 4 waves
// of a workgroup take 4 consecutive tokens of that group.  Otherwise one workgroup takes
// one token and its waves take the groups (adjacent rows of one token).
template <int D, bool kGroupPerXcd>
__global__ __launch_bounds__(512) void k_attn_prefill(AttnArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    const int wave = wave_index();
    const int hpg = a.Hq / a.Hkv;
    int64_t r;
    int g;
    if (!wave_row_group<kGroupPerXcd>(a, r, g))
        return;  // waves never synchronise with each other
    const int64_t t = a.q_start + r;
    const int64_t c = t / a.B;
    const int nvalid = (int)((c + 1 < a.k) ? c + 1 : a.k);
    // History-sliced launches: launch `slice` covers the blocks [slice*W, (slice+1)*W) of a
    // row's history, so the launch's rows gather from one W-block range of the cache.  W is
    // slice_blocks for histories of up to 16 such ranges; a longer history is cut into
    // long_slices ranges of its own length instead (a row would otherwise park its state at
    // more boundaries than it has entries to gather between them).  A row takes part in
    // launches 0 .. c/W (the last one also holds its own block c).  Rows with a short history
    // (c < 2k) are attended in one pass, in launch c/W.  Every choice depends only on the row's
    // own c and selection, so a row's bits do not depend on its launch's other rows.
    int64_t W = a.slice_blocks;
    if (W > 0 && c + 1 > kMaxBaseSlices * W)
        W = (c + a.long_slices) / a.long_slices;  // ceil((c + 1) / long_slices)
    const int64_t last = W > 0 ? c / W : 0;
    if (W > 0 && a.slice > last)
        return;
    const bool sliced = W > 0 && c >= 2 * (int64_t)a.k;
    if (W > 0 && !sliced && a.slice != last)
        return;

    int e_lo = 0, e_hi = nvalid;
    bool first = true;
    if (sliced) {
        // entries of this launch: the idx row is ascending, so the blocks in [lo, hi) are a
        // contiguous run of entries; the row's first launch with entries is the one holding its
        // first entry's block
        const int64_t lo = (int64_t)a.slice * W;
        const int64_t hi = a.slice == last ? c + 1 : lo + W;
        const int32_t *row = a.idx + r * a.k;
        const int lane = threadIdx.x & 63;
        int below_lo = 0, below_hi = 0;
        int32_t head = 0;
        for (int e0 = 0; e0 < nvalid; e0 += 256) {  // four loads in flight per lane
            int32_t b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * 64 + lane;
                b[u] = row[e < nvalid ? e : 0];
            }
            if (e0 == 0)
                head = b[0];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool in = e0 + u * 64 + lane < nvalid && b[u] >= 0;
                below_lo += (in && b[u] < lo) ? 1 : 0;
                below_hi += (in && b[u] < hi) ? 1 : 0;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            below_lo += __shfl_xor(below_lo, o);
            below_hi += __shfl_xor(below_hi, o);
        }
        const int64_t first_slice = (int64_t)__shfl(head, 0) / W;  // lane 0 read entry 0
        if (a.slice < first_slice)
            return;  // no entries yet: the state starts in a later launch
        e_lo = below_lo;
        e_hi = a.slice == last ? nvalid : below_hi;
        first = a.slice == first_slice;
        if (!first && a.slice < last && e_lo == e_hi)
            return;  // nothing in this range: the parked state stays as it is
    }

    bf16x8 qf[D / 32];
    load_q<D>(a.q + (r * a.Hq + (int64_t)g * hpg) * D, hpg, qf);
    WaveState<D> st;
    if (first)
        init_state<D>(st);
    else
        load_state<D>(st, a.state + state_offset(a, r, g));
    const SparseTokens src{a.idx + r * a.k, e_lo, e_hi, t, c, a.B, entry_window<D>(lds)};
    attend_range<D>(Bf16Rows{a.kc + (int64_t)g * D, a.vc + (int64_t)g * D}, a.Hkv, src,
                    QRegs<D>{qf}, a.scale_log2, lds + wave * attn_vbuf_elems(D), st);

    if (!sliced || a.slice == last)
        store_row<D>(st, a, r, g, hpg);
    else
        save_state<D>(st, a.state + state_offset(a, r, g));
}

// ---- resident prefill: the history ranges of the sliced prefill in one launch ------------
// The sliced prefill parks every row's softmax state between its range launches (13 KB per row
// and group each way) and reloads its query.  Here a persistent grid of exactly the resident
// workgroups keeps each row's state in the wave's registers across the ranges: the waves of one
// XCD take a batch of nw_x consecutive rows of the XCD's KV group (the R = 8 / Hkv XCDs of a
// group split the group's batch of R * nw_x rows), attend range 0 of all of them, then range 1,
// and so on, and move to their next batch.  Between ranges a wave waits, up to a bounded time,
// until most waves of its XCD have finished the previous range, so the XCD's L2 holds one
// range of its group's K/V rows at a time; the wait only orders the work for the caches (it
// guards no data), so a wave that stops waiting at the bound still computes the same result.
// Each row attends the same entries per range, in the same steps, as in the sliced launches,
// so its bits equal the sliced prefill's.
constexpr int kResidentRanges = 16;  // ranges of the longest history the resident prefill takes
constexpr int kResidentSpin = 4096;  // polls per wait (a few ms) before a wave goes on anyway
// A wave starts range s once three quarters of its XCD's waves of the batch have finished range
// s - 1 (waiting for more lets the slowest rows hold everyone up; for fewer, the L2 holds
// two ranges).  128K prefill, range width x share waited for: 2560 blocks x 3/4 111.3 ms,
// x 2/3 111.6, x 4/5 112.2, x 1/2 139.8 (3072 blocks); 2048 x 3/4 116.0; 1024 x 3/4 137.4
// x 15/16 145.7; 4096 x 3/4 123.3; waiting for the range before the previous one, 157.5.
constexpr int kResidentSlack = 4;     // a wave waits for all but 1/slack of them

// Entries of `row` (nvalid ascending blocks, -1 past the valid ones) below block `lim`.
__device__ __forceinline__ int entries_below(const int32_t *row, int nvalid, int64_t lim)
{
    const int lane = threadIdx.x & 63;
    int n = 0;
    for (int e0 = 0; e0 < nvalid; e0 += 256) {  // four loads in flight per lane
        int32_t b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * 64 + lane;
            b[u] = row[e < nvalid ? e : 0];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool in = e0 + u * 64 + lane < nvalid && b[u] >= 0;
            n += (in && b[u] < lim) ? 1 : 0;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        n += __shfl_xor(n, o);
    return n;
}

// A wave-uniform value kept in scalar registers.
__device__ __forceinline__ int uni(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int64_t uni(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Progress words of an XCD's waves: wave i stores, after each range it finishes, the number
// of ranges it has finished since the launch (each wave its own word, so no two waves write
// the same address).  A wave waits, up to kResidentSpin polls, until at least `need` of the
// nw words reach `target`.
__device__ __forceinline__ void resident_wait(const uint32_t *prog, int nw, uint32_t target,
                                              int need)
{
    const int lane = threadIdx.x & 63;
    for (int i = 0; i < kResidentSpin; ++i) {
        int n = 0;
        for (int w = lane; w < nw; w += 64)
            n += __hip_atomic_load(prog + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target
                     ? 1
                     : 0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            n += __shfl_xor(n, o);
        if (uni(n) >= need)
            return;
        __builtin_amdgcn_s_sleep(8);
    }
}

// a.state: one progress word per wave (8 XCDs x 4 a.slice, zero at launch); a.slice: the
// workgroups of one XCD (the grid is 8 times that); a.slice_blocks: the range width W, every
// row's history within kResidentRanges ranges.
template <int D>
__global__ __launch_bounds__(512) void k_attn_prefill_resident(AttnArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    const int wave = wave_index();
    const int hpg = a.Hq / a.Hkv;
    const int R = 8 / a.Hkv;                 // XCDs per KV group
    const int x = blockIdx.x & 7;            // this workgroup's XCD
    const int g = x / R, h = x % R;
    const int nw_x = a.slice * 4;            // waves per XCD
    const int lw = (int)(blockIdx.x >> 3) * 4 + wave;
    const int64_t W = a.slice_blocks;
    uint32_t *prog = reinterpret_cast<uint32_t *>(a.state) + (int64_t)x * nw_x;
    const int64_t per_batch = (int64_t)R * nw_x;
    uint32_t done = 0;                       // ranges of the earlier batches
    for (int64_t b = 0; b * per_batch < a.rows; ++b) {
        // this XCD's rows of the batch, longest history first
        const int64_t j0 = b * per_batch + (int64_t)h * nw_x;
        const int64_t left = (int64_t)a.rows - j0;
        const int nval = (int)(left < 0 ? 0 : (left < nw_x ? left : nw_x));
        const int64_t c_max = (a.q_start + (int64_t)a.rows - 1 - b * per_batch) / a.B;
        const int S = (int)(c_max / W) + 1;  // ranges of the batch (its longest row)
        const bool live = lw < nval;
        const int64_t r = uni((int64_t)a.rows - 1 - (j0 + lw));
        const int64_t t = a.q_start + r;
        const int64_t c = uni(live ? t / a.B : (int64_t)0);
        const int nvalid = (int)((c + 1 < a.k) ? c + 1 : a.k);
        const int last = uni((int)(c / W));
        const bool sliced = c >= 2 * (int64_t)a.k;
        const int32_t *row = a.idx + (live ? r : 0) * a.k;
        const int first_slice = uni(live && sliced ? (int)((int64_t)row[0] / W) : last);
        WaveState<D> st;
        init_state<D>(st);
        int e_lo = 0;
        for (int s = 0; s < S; ++s) {
            // most of the XCD's waves of this batch are done with range s - 1
            if (s > 0 && nval > 0)
                resident_wait(prog, nw_x, done + (uint32_t)s, nval - nval / kResidentSlack);
            if (live && s >= first_slice && s <= last) {
                const int e_hi =
                    uni(s == last ? nvalid : entries_below(row, nvalid, (int64_t)(s + 1) * W));
                if (e_hi > e_lo) {
                    bf16x8 qf[D / 32];
                    load_q<D>(a.q + (r * a.Hq + (int64_t)g * hpg) * D, hpg, qf);
                    const SparseTokens src{row, e_lo, e_hi, t, c, a.B, entry_window<D>(lds)};
                    attend_range<D>(Bf16Rows{a.kc + (int64_t)g * D, a.vc + (int64_t)g * D},
                                    a.Hkv, src, QRegs<D>{qf}, a.scale_log2,
                                    lds + wave * attn_vbuf_elems(D), st);
                }
                e_lo = e_hi;
            }
            if (live && (threadIdx.x & 63) == 0)
                __hip_atomic_store(prog + lw, done + (uint32_t)s + 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (live)
            store_row<D>(st, a, r, g, hpg);
        done += (uint32_t)S;
    }
}

typedef __attribute__((ext_vector_type(2))) float f2v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;

// O^T += V^T P^T for one 32-position step of the sliding-window kernel (V rows [slot][kLd] at
// `vs`): the transposing reads of two MFMA operands are issued together and waited for inside
// the asm block.  Written as asm because the compiler has no memory-operand information for
// the ds_read_b64_tr_b16 builtin and so waits for every global-to-LDS copy in flight, the
// next tile's included, before the first of them; these reads only touch the current tile.
template <int D, int kLd>
__device__ __forceinline__ void swa_pv_step(const uint16_t *vs, bf16x8 pf, f32x4 (&acc)[D / 16])
{
    static_assert((D / 16) % 2 == 0 && (D / 16 - 1) * 32 + 64 * kLd < 65536, "ds offsets");
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    // tr_quad's address for d0 = 0; d0 and the second 16 slots are immediate offsets
    const uint16_t *p = vs + (q4 * 4 + (col >> 2)) * kLd + 4 * (col & 3);
    const uint32_t addr =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t *)p;
    typedef __attribute__((ext_vector_type(8))) short s16x8;
#pragma unroll
    for (int mt = 0; mt < D / 16; mt += 2) {
        s16x4 a0, a1, b0, b1;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
            "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
            "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
            : "v"(addr), "i"(mt * 32), "i"(mt * 32 + 32 * kLd), "i"(mt * 32 + 32),
              "i"(mt * 32 + 32 + 32 * kLd)
            : "memory");
        const s16x8 va = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const s16x8 vb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[mt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, va), pf, acc[mt]);
        acc[mt + 1] = mfma_16x16x32(__builtin_bit_cast(bf16x8, vb), pf, acc[mt + 1]);
    }
}

// Gated sliding-window attention, query-tiled: neighbouring queries share all but one of
// their window positions, so a workgroup takes 16 consecutive queries of one KV group and each
// 32-position step of the group's K and V rows is staged once in LDS for all of them.  One wave
// per head; the group's heads are split over a few workgroups (blockIdx / Hkv % parts), each
// staging the same tiles.  The wave's arithmetic is the sparse kernel's with the MFMA N
// dimension taken as the 16 queries of one head instead of the 16 heads of one query:
//   S^T[pos][query] = K_tile . Q_h^T (K rows from LDS as the A operand),
//   online softmax per query (= lane % 16), O^T[d][query] += V_tile^T . P^T.
// Positions outside [t - window + 1, t] of a query are masked.  Group = blockIdx % Hkv, so
// with Hkv dividing 8 each XCD's L2 holds one group's rows.  The tile is double-buffered and
// filled by direct global-to-LDS loads (global_load_lds_dwordx4: lane l of an instruction
// writes 16 bytes at base + 16 l), so the next step's rows stream in while the current step is
// computed, without holding registers.  A step's tile is 2 x 32 rows of kLd/8 16-byte pieces
// (a whole number of 64-piece instructions); the pad pieces of a row reload the row's first
// piece and are never read.
template <int D>
__global__ __launch_bounds__(1024) void k_swa_tiled(AttnArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    // row stride (elements): 16-byte aligned rows, padded by 16 so the transposing V reads are
    // free of bank conflicts (5.87 ms vs 6.05 ms with a pad of 8 at 128K)
    constexpr int kLd = D + 16;
    constexpr int kTile = 2 * kSlots * kLd;  // K then V rows of one step
    const int hpg = a.Hq / a.Hkv;
    const int wave = wave_index(), lane = threadIdx.x & 63;
    const int nwaves = (int)(blockDim.x >> 6);      // heads per workgroup
    const int hs = (hpg + nwaves - 1) / nwaves;     // workgroups per (query tile, group)
    const int g = (int)(blockIdx.x % (unsigned)a.Hkv);
    const int part = (int)((blockIdx.x / (unsigned)a.Hkv) % (unsigned)hs);
    const int64_t r0 = (int64_t)(blockIdx.x / (unsigned)(a.Hkv * hs)) * 16;  // first query row
    const int col = lane & 15, q4 = lane >> 4;
    const int nq = a.rows - r0 < 16 ? (int)(a.rows - r0) : 16;
    const int hw = part * nwaves + wave;            // this wave's head within the group
    const bool has_head = hw < hpg;
    const int h = g * hpg + (has_head ? hw : 0);
    const int64_t t0 = a.q_start + r0;
    const int64_t t_last = t0 + nq - 1;
    const int64_t ks0 = t0 - a.window + 1 > 0 ? t0 - a.window + 1 : 0;
    const int nsteps = (int)((t_last - ks0 + kSlots) / kSlots);
    const int64_t row_elems = (int64_t)a.Hkv * D;
    const float neg_inf = -__builtin_inff();

    // Q of head h for the tile's queries (B operand: query col, dims 8 q4 + 32 kk)
    bf16x8 qf[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (col < nq)
            v = load16(a.q + ((r0 + col) * a.Hq + h) * D + kk * 32 + q4 * 8);
        if (a.scale_log2 < 0.f)
            v ^= 0x80008000u;  // -q, so the scores come out negated (exactly)
        qf[kk] = as_bf16x8(v);
    }
    WaveState<D> st;
    init_state<D>(st);
    const int64_t tq = t0 + col;  // this lane's query position
    // the window, at most every position up to the tile's last query (positions < 2^31)
    const int wnd = (int)(a.window < t_last + 1 ? a.window : t_last + 1);
    const uint32_t win = col < nq ? (uint32_t)wnd : 0u;
    // |scale| (at least the smallest normal float, so that a zero scale still gives -inf for
    // masked scores and equal weights for the others)
    const float scale_abs = fmaxf(__builtin_fabsf(a.scale_log2), 1.17549435e-38f);

    constexpr int kPpr = kLd / 8;                       // 16-byte pieces per LDS row
    constexpr int kTilePieces = 2 * kSlots * kPpr;
    // K pieces fill whole instructions, so each instruction reads only K or only V rows
    static_assert((kSlots * kPpr) % 64 == 0, "whole instructions");
    // The wave's first kPre DMA instructions (i = wave + u * nwaves), described once: this
    // lane's byte offset from the step's first row, voff = row * row_bytes + piece offset
    // (the step's first row and K or V come from a wave-uniform base).  Rows past t_last
    // (only in the last step; they are masked below) must not be read: the offset is capped
    // at the last piece of the group's part of row t_last, which every larger offset exceeds.
    constexpr int kPre = 4;
    constexpr int kInstr = kTilePieces / 64;
    const uint32_t row_bytes = (uint32_t)(row_elems * sizeof(uint16_t));
    uint32_t voff[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int i = wave + u * nwaves;
        const int pc = (i < kInstr ? i : 0) * 64 + lane;
        const int rem = pc % (kSlots * kPpr);
        const int slot = rem / kPpr, piece = rem - slot * kPpr;
        voff[u] = (uint32_t)slot * row_bytes + (uint32_t)(piece < D / 8 ? piece : 0) * 16u;
    }
    auto dma = [&](int step, uint16_t *buf) {
        const int64_t k0 = ks0 + (int64_t)step * kSlots;
        const uint32_t cap = (uint32_t)(t_last - k0) * row_bytes + (uint32_t)(D * 2 - 16);
        const int64_t roff = k0 * row_elems + g * D;
        const char *kb = reinterpret_cast<const char *>(a.kc + roff);
        const char *vb = reinterpret_cast<const char *>(a.vc + roff);
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const int i = wave + u * nwaves;
            if (i < kInstr) {
                const char *base = i * 64 >= kSlots * kPpr ? vb : kb;
                const uint32_t off = voff[u] < cap ? voff[u] : cap;
                __builtin_amdgcn_global_load_lds(
                    (const void __attribute__((address_space(1))) *)(base + off),
                    (void __attribute__((address_space(3))) *)(buf + i * 64 * 8), 16, 0, 0);
            }
        }
        // small workgroups issue the remaining instructions here
        for (int i = wave + kPre * nwaves; i < kTilePieces / 64; i += nwaves) {
            const int pc = i * 64 + lane;
            const int which = pc / (kSlots * kPpr);
            const int rem = pc - which * kSlots * kPpr;
            const int slot = rem / kPpr, piece = rem - slot * kPpr;
            int64_t sp = k0 + slot;
            if (sp > t_last)
                sp = t_last;
            const uint16_t *src = (which ? a.vc : a.kc) + sp * row_elems + (int64_t)g * D +
                                  (piece < D / 8 ? piece : 0) * 8;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)src,
                (void __attribute__((address_space(3))) *)(buf + i * 64 * 8), 16, 0, 0);
        }
    };
    // steps whose every position lies in every query's window (k0 + 31 <= t0 and
    // k0 > t_last - wnd, with all 16 queries present) skip the mask
    int full0 = 0, full1 = -1;
    if (nq == 16) {
        const int64_t lo = t_last - wnd + 1 - ks0, hi = t0 - (kSlots - 1) - ks0;
        full0 = lo <= 0 ? 0 : (int)((lo + kSlots - 1) / kSlots);
        full1 = hi < 0 ? -1 : (int)(hi / kSlots);
    }
    full0 = __builtin_amdgcn_readfirstlane(full0);
    full1 = __builtin_amdgcn_readfirstlane(full1);
    const float pinf = opaque_pinf();
    dma(0, lds);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed in LDS
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
        const int64_t k0 = ks0 + (int64_t)step * kSlots;
        const bool more = step + 1 < nsteps;
        if (more)
            dma(step + 1, lds + ((step + 1) & 1) * kTile);
        const uint16_t *ks = lds + (step & 1) * kTile;
        const uint16_t *vs = ks + kSlots * kLd;

        // S^T for positions 0-15 and 16-31 of the tile
        f32x4 sc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            sc[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const u32x4 kv =
                    *reinterpret_cast<const u32x4 *>(ks + (hh * 16 + col) * kLd + kk * 32 + q4 * 8);
                sc[hh] = mfma_16x16x32(as_bf16x8(kv), qf[kk], sc[hh]);
            }
        }
        // online softmax (base 2) per query; lane holds positions 16 hh + 4 q4 + r of query col.
        // Only a tile's first and last steps hold positions outside some query's window: there
        // rel = position - query must lie in [1 - window, 0], i.e. rel + window - 1 in
        // [0, win) as an unsigned compare (win = 0 for the lanes of absent queries), and the
        // other scores become -inf.  The scale is applied with the exponent's subtraction
        // (with a negative scale the query was negated, so the maximum commutes with |scale|).
        if (step < full0 || step > full1) {
            const int rel0 = (int)(k0 - tq) + q4 * 4 + wnd - 1;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!((uint32_t)(rel0 + hh * 16 + r) < win))
                        sc[hh][r] = neg_inf;
        }
        const float mloc =
            max_med3(max_med3(max_med3(sc[0][0], sc[0][1], pinf), max_med3(sc[0][2], sc[0][3], pinf), pinf),
                     max_med3(max_med3(sc[1][0], sc[1][1], pinf), max_med3(sc[1][2], sc[1][3], pinf), pinf),
                     pinf);
        // the running maximum moves only when a step raises it by more than kLazyMax (log2
        // units), so most steps skip the rescale; the weights exp2(x - m) stay below
        // 2^kLazyMax, and the output and lse use the same m as the sums
        const float m_row = fmaxf(st.m, max_across_rows_swap(mloc, pinf) * scale_abs);
        const float m_new = m_row > st.m + kLazyMax ? m_row : st.m;
        const bool any = m_new != neg_inf;
        const float alpha = any ? fast_exp2(st.m - m_new) : 1.0f;
        const float m_sub = any ? -m_new : 0.f;  // masked scores stay -inf, their weights 0
        float pe[2][4];
        f2v pv[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pe[hh][r] = fast_exp2(__builtin_fmaf(sc[hh][r], scale_abs, m_sub));
        // the weights PV uses are the bf16 ones; normalise by their sum too (a bf16 pair is
        // summed by one dot product with (1, 1): the products are exact)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            pv[c] = f2v{pe[c >> 1][2 * (c & 1)], pe[c >> 1][2 * (c & 1) + 1]};
        float psum = 0.f, psum32 = 0.f;
        u32x4 pw;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x2v b = __builtin_convertvector(pv[c], bf16x2v);
            pw[c] = __builtin_bit_cast(uint32_t, b);
            psum = __builtin_amdgcn_fdot2_f32_bf16(b, bf16x2v{(__bf16)1.0f, (__bf16)1.0f}, psum,
                                                   false);
            psum32 += pv[c][0] + pv[c][1];
        }
        st.l = st.l * alpha + psum;
        st.l32 = st.l32 * alpha + psum32;
        st.m = m_new;
        if (__ballot(alpha != 1.0f)) {  // no lane's maximum moved: nothing to rescale
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    st.acc[mt][r] *= alpha;
        }
        // O^T += V^T P^T: A[m = d][k = position perm(8 q4 + j)] from the staged V rows
        swa_pv_step<D, kLd>(vs, as_bf16x8(pw), st.acc);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the next tile has landed
        __syncthreads();                 // the next tile is complete; this one is no longer read
    }

    // lane holds O^T[d = 16 mt + 4 q4 + i][query col] of head h
    const float l = sum_across_rows(st.l);
    const float l32 = sum_across_rows(st.l32);
    if (has_head && col < nq) {
        const int64_t row = (r0 + col) * a.Hq + h;
        const float f = sigmoid_f32(bf16_bits_to_f32(a.gate[row])) / l;
        uint16_t *o = a.out + row * D + q4 * 4;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
            uint2 w;
            w.x = pack_bf16x2(st.acc[mt][0] * f, st.acc[mt][1] * f);
            w.y = pack_bf16x2(st.acc[mt][2] * f, st.acc[mt][3] * f);
            *reinterpret_cast<uint2 *>(o + mt * 16) = w;
        }
        if (a.lse && q4 == 0)
            a.lse[row] = (st.m + fast_log2(l32)) * 0.6931471805599453f;
    }
}

// Decode, split over the selection: a workgroup takes one (sequence, KV group) and nw
// consecutive splits of its selection entries, one split per wave.  The waves' partial
// softmax states are combined in LDS (in wave order, so the sums do not depend on timing)
// and the workgroup writes one partial state; k_attn_decode_merge combines the workgroups'.
template <int D, bool kFp8>
__global__ __launch_bounds__(512) void k_attn_decode_part(AttnArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    const int wave = wave_index(), lane = threadIdx.x & 63;
    const int nw = blockDim.x >> 6;
    const int col = lane & 15, q4 = lane >> 4;
    const int s = blockIdx.y / a.Hkv;
    const int g = blockIdx.y - s * a.Hkv;
    const int split = blockIdx.x * nw + wave;
    const int64_t t = a.qpos.v[s];
    const int64_t c = t / a.B;
    const int nvalid = (int)((c + 1 < a.k) ? c + 1 : a.k);
    const int e0 = split * a.entries_per_split;
    const int e1 = min(e0 + a.entries_per_split, nvalid);
    const int hpg = a.Hq / a.Hkv;

    WaveState<D> st;
    init_state<D>(st);
    const int64_t base = (int64_t)s * a.cache_seq_stride + (int64_t)g * D;
    const uint16_t *qg = a.q + ((int64_t)s * a.Hq + (int64_t)g * hpg) * D;
    bf16x8 qf[D / 32];
    if constexpr (kFp8)
        load_q_perm<D>(qg, hpg, qf);
    else
        load_q<D>(qg, hpg, qf);
    if (e0 < e1) {
        const SparseTokens src{a.idx + (int64_t)s * a.k, e0, e1, t, c, a.B, entry_window<D>(lds)};
        uint16_t *vs = lds + wave * attn_vbuf_elems(D);
        if constexpr (kFp8) {
            const int64_t sb = (int64_t)s * a.scale_seq_stride * a.Hkv + g;
            const Fp8Rows rows{a.kq + base, a.vq + base, a.ksc + sb, a.vsc + sb};
            attend_range<D>(rows, a.Hkv, src, QRegs<D>{qf}, a.scale_log2, vs, st);
        } else {
            Bf16StreamRows rows;
            rows.Kg = a.kc + base;
            rows.Vg = a.vc + base;
            attend_range<D>(rows, a.Hkv, src, QRegs<D>{qf}, a.scale_log2, vs, st);
        }
    }

    // combine the waves: (max, sums) per (wave, head), then every wave's accumulators scaled
    // to the workgroup's maximum, summed over the waves in order by the whole workgroup.
    // The LDS of the attention (V buffers, windows) is reused: 64 D + 192 bytes per wave.
    const float l = sum_across_rows(st.l);
    const float l32 = sum_across_rows(st.l32);
    float *accb = reinterpret_cast<float *>(lds);  // [nw][64 lanes][D / 4]
    float *mlb = accb + nw * 64 * (D / 4);          // [nw][16 heads][3]
    __syncthreads();  // every wave is done with its V buffer and window
    if (q4 == 0) {
        mlb[(wave * 16 + col) * 3 + 0] = st.m;
        mlb[(wave * 16 + col) * 3 + 1] = l;
        mlb[(wave * 16 + col) * 3 + 2] = l32;
    }
    __syncthreads();
    const float neg_inf = -__builtin_inff();
    float M = neg_inf;
    for (int w = 0; w < nw; ++w)
        M = fmaxf(M, mlb[(w * 16 + col) * 3]);
    const float f = st.m == neg_inf ? 0.f : fast_exp2(st.m - M);
    float *mine = accb + (wave * 64 + lane) * (D / 4);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        *reinterpret_cast<f32x4 *>(mine + mt * 4) = st.acc[mt] * f;
    __syncthreads();
    const int64_t slot0 = ((int64_t)s * a.npart + blockIdx.x) * a.Hq + (int64_t)g * hpg;
    // value v = (head v / D, dim v % D): consecutive threads write consecutive dims
    for (int v = threadIdx.x; v < hpg * D; v += nw * 64) {
        const int head = v / D, dim = v - head * D;
        const int src = (((dim & 15) >> 2) * 16 + head) * (D / 4) + (dim >> 4) * 4 + (dim & 3);
        float o = 0.f;
        for (int w = 0; w < nw; ++w)
            o += accb[w * 64 * (D / 4) + src];
        a.part_o[(slot0 + head) * D + dim] = o;
    }
    if ((int)threadIdx.x < hpg) {
        const int head = (int)threadIdx.x;
        float m = neg_inf, ls = 0.f, l32s = 0.f;
        for (int w = 0; w < nw; ++w)
            m = fmaxf(m, mlb[(w * 16 + head) * 3]);
        for (int w = 0; w < nw; ++w) {
            const float mw = mlb[(w * 16 + head) * 3];
            const float fw = mw == neg_inf ? 0.f : fast_exp2(mw - m);
            ls += mlb[(w * 16 + head) * 3 + 1] * fw;
            l32s += mlb[(w * 16 + head) * 3 + 2] * fw;
        }
        a.part_ml[(slot0 + head) * 3 + 0] = m;
        a.part_ml[(slot0 + head) * 3 + 1] = ls;
        a.part_ml[(slot0 + head) * 3 + 2] = l32s;
    }
}

// Exact merge of the workgroups' partial states of one (sequence, head), then the gate.
// One thread per output dimension.  Every thread issues all its loads at once (its
// dimension's partial outputs, clamped to the parts present so no branch holds them back,
// and every part's (max, sums) as vector loads of one address: as scalar loads the compiler
// waited for each before computing with it), so the merge waits for memory once and needs
// no barrier.
constexpr int kMaxSplits = 32;  // decode_split_plan never makes more
#ifndef SGQA_DECODE_WAVES
#define SGQA_DECODE_WAVES 8
#endif
constexpr int kDecodeWaves = SGQA_DECODE_WAVES;  // splits (waves) per decode workgroup
constexpr int kMaxParts = (kMaxSplits + kDecodeWaves - 1) / kDecodeWaves;  // workgroups

__global__ __launch_bounds__(256) void k_attn_decode_merge(AttnArgs a)
{
    const int s = blockIdx.y, h = blockIdx.x;
    const int D = a.d, ns = a.npart, tid = threadIdx.x;
    const float neg_inf = -__builtin_inff();
    const int64_t base = (int64_t)s * ns * a.Hq + h;  // slot of part 0
    const int64_t step = (int64_t)a.Hq * D;
    const float *po = a.part_o + base * D + (tid < D ? tid : D - 1);
    int lz;  // a zero the compiler cannot see through, so the (max, sums) loads stay vector
    asm volatile("v_mov_b32 %0, 0" : "=v"(lz));
    float ov[kMaxParts], mw[kMaxParts], lw[kMaxParts], l32w[kMaxParts];
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
        const int ic = i < ns ? i : ns - 1;
        ov[i] = po[ic * step];
        const float *ml = a.part_ml + (base + (int64_t)ic * a.Hq) * 3 + lz;
        mw[i] = ml[0];
        lw[i] = ml[1];
        l32w[i] = ml[2];
    }
    const uint16_t gbits = a.gate[(int64_t)s * a.Hq + h];
    float M = neg_inf;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i)
        if (i < ns)
            M = fmaxf(M, mw[i]);
    float Lsum = 0.f, L32 = 0.f, o = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
        if (i < ns) {
            const float w = mw[i] == neg_inf ? 0.f : fast_exp2(mw[i] - M);
            Lsum += lw[i] * w;
            L32 += l32w[i] * w;
            o += ov[i] * w;
        }
    }
    if (tid < D) {
        const float gsig = sigmoid_f32(bf16_bits_to_f32(gbits));
        a.out[((int64_t)s * a.Hq + h) * D + tid] = (uint16_t)f32_to_bf16_bits(o * (gsig / Lsum));
    }
    if (a.lse && tid == 0)
        a.lse[(int64_t)s * a.Hq + h] = (M + fast_log2(L32)) * 0.6931471805599453f;
}

void decode_split_plan(int k, int B, int &nsplit, int &entries_per_split)
{
    const int eps = kSlots / B;  // entries per 32-slot step
    int per = (k + 31) / 32;     // aim for 32 splits: 2048 waves at the real shape, one per
                                 // SIMD slot (16 and 64 splits measured 15 % slower)
    per = ((per + eps - 1) / eps) * eps;
    entries_per_split = per;
    nsplit = (k + per - 1) / per;
}

template <int D>
static hipError_t launch_prefill_d(const AttnArgs &a, hipStream_t stream)
{
    // Group-per-XCD mapping whenever the groups divide the 8 XCDs (measured 17 % faster
    // than one-token-per-workgroup on the 128K prefill); the other mapping otherwise.
    if (8 % a.Hkv == 0) {
        const int R = 8 / a.Hkv;
        const int64_t ntiles = ((int64_t)a.rows + 3) / 4;
        const int64_t nwg = (ntiles + R - 1) / R * 8;
        const size_t lds = (size_t)4 * attn_wave_lds(D);
        hipLaunchKernelGGL((k_attn_prefill<D, true>), dim3((unsigned)nwg), dim3(256), lds, stream,
                           a);
    } else {
        const size_t lds = (size_t)a.Hkv * attn_wave_lds(D);
        hipLaunchKernelGGL((k_attn_prefill<D, false>), dim3((unsigned)a.rows), dim3(64 * a.Hkv),
                           lds, stream, a);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_swa_d(const AttnArgs &a, hipStream_t stream)
{
    // The group's heads are split over two workgroups (8 waves each at 16 heads), so that two
    // of them share a CU and one computes while the other waits at its step barrier
    // (6.37 -> 6.04 ms at 128K; four workgroups of 4 waves: 7.25 ms)
    const int hpg = a.Hq / a.Hkv;
    const int hs = hpg >= 2 ? 2 : 1;
    const int nw = (hpg + hs - 1) / hs;
    const int64_t nwg = ((int64_t)a.rows + 15) / 16 * a.Hkv * hs;
    const size_t lds = (size_t)2 * 2 * kSlots * (D + 16) * sizeof(uint16_t);
    hipLaunchKernelGGL(k_swa_tiled<D>, dim3((unsigned)nwg), dim3(64 * nw), lds, stream, a);
    return hipGetLastError();
}

// Sliced prefill: rows in chunks that fit the workspace; each chunk in one launch per
// slice_blocks-block range of history, up to the range holding the chunk's last own block.
template <int D>
static hipError_t launch_prefill_sliced(const AttnArgs &a0, hipStream_t stream)
{
    const int64_t per_row = (int64_t)a0.Hkv * 64 * a0.state_stride * sizeof(float);
    int64_t chunk = a0.state_bytes / per_row;
    if (chunk > a0.rows)
        chunk = a0.rows;
    for (int64_t r0 = 0; r0 < a0.rows; r0 += chunk) {
        AttnArgs a = a0;
        const int64_t n = a0.rows - r0 < chunk ? a0.rows - r0 : chunk;
        a.rows = (int32_t)n;
        a.q_start = a0.q_start + r0;
        a.q = a0.q + r0 * a0.Hq * D;
        a.gate = a0.gate + r0 * a0.Hq;
        a.idx = a0.idx + r0 * a0.k;
        a.out = a0.out + r0 * a0.Hq * D;
        a.lse = a0.lse ? a0.lse + r0 * a0.Hq : nullptr;
        // rows of up to kMaxBaseSlices ranges end in launch c / slice_blocks; longer ones in
        // launch long_slices - 1 or earlier
        const int64_t c_first = a.q_start / a0.B, c_last = (a.q_start + n - 1) / a0.B;
        const int64_t c_short_max = kMaxBaseSlices * a0.slice_blocks - 1;
        int64_t nsl = 0;
        if (c_first <= c_short_max)  // rows of the base ranges
            nsl = (c_last < c_short_max ? c_last : c_short_max) / a0.slice_blocks + 1;
        if (c_last > c_short_max && a0.long_slices > nsl)  // rows cut into long_slices ranges
            nsl = a0.long_slices;
        for (int64_t sl = 0; sl < nsl; ++sl) {
            a.slice = (int32_t)sl;
            hipError_t e = launch_prefill_d<D>(a, stream);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

int decode_parts(int nsplit)
{
    const int nw = nsplit < kDecodeWaves ? nsplit : kDecodeWaves;
    return (nsplit + nw - 1) / nw;
}

template <int D>
static hipError_t launch_decode_d(const AttnArgs &a0, hipStream_t stream)
{
    if (a0.nsplit < 1 || a0.nsplit > kMaxSplits)
        return hipErrorInvalidValue;  // the merge holds at most kMaxParts partial states
    AttnArgs a = a0;
    const int nw = a.nsplit < kDecodeWaves ? a.nsplit : kDecodeWaves;
    a.npart = decode_parts(a.nsplit);
    if (a.npart > kMaxParts)
        return hipErrorInvalidValue;  // the merge holds at most kMaxParts partial states
    // the V buffers and windows of the waves hold their combine buffers (64 D + 192 B each)
    static_assert(attn_wave_lds(D) >= (size_t)64 * D + 192, "decode combine buffer");
    const size_t lds = (size_t)nw * attn_wave_lds(D);
    const dim3 grid((unsigned)a.npart, (unsigned)(a.rows * a.Hkv));
    if (a.kq)
        hipLaunchKernelGGL((k_attn_decode_part<D, true>), grid, dim3(64 * nw), lds, stream, a);
    else
        hipLaunchKernelGGL((k_attn_decode_part<D, false>), grid, dim3(64 * nw), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const unsigned nt = (unsigned)((a.d + 63) / 64 * 64);
    hipLaunchKernelGGL(k_attn_decode_merge, dim3((unsigned)a.Hq, (unsigned)a.rows), dim3(nt), 0,
                       stream, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t *p, int n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n)
        p[i] = 0u;
}

// The resident prefill over rows [0, a0.rows), whose histories span at most kResidentRanges
// ranges of a0.resident_blocks blocks: one launch of as many workgroups as are resident at
// once (occupancy x CUs), after a fill kernel clears the waves' progress words in the
// workspace.  Returns hipErrorNotSupported when the workspace cannot hold the progress words.
template <int D>
static hipError_t launch_prefill_resident(const AttnArgs &a0, hipStream_t stream)
{
    const size_t lds = (size_t)4 * attn_wave_lds(D);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attn_prefill_resident<D>, 256,
                                                         lds);
    if (e != hipSuccess)
        return e;
    const int per_xcd = per_cu * (cus / 8);
    const int words = 8 * per_xcd * 4;  // one progress word per wave
    if (per_xcd < 1 || a0.state_bytes < (int64_t)words * (int64_t)sizeof(uint32_t))
        return hipErrorNotSupported;
    AttnArgs a = a0;
    a.slice = per_xcd;
    a.slice_blocks = a0.resident_blocks;
    uint32_t *prog = reinterpret_cast<uint32_t *>(a.state);
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       prog, words);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_attn_prefill_resident<D>, dim3((unsigned)(8 * per_xcd)), dim3(256), lds,
                       stream, a);
    return hipGetLastError();
}

// With a workspace: the rows whose histories span at most kResidentRanges resident ranges
// (a prefix of the rows) go to the resident prefill when the KV groups divide the 8 XCDs, the
// others to the sliced launches; which path a row takes depends only on its own history.
template <int D>
static hipError_t launch_prefill_ws(const AttnArgs &a0, hipStream_t stream)
{
    int64_t n_res = 0;
    if (a0.resident_blocks > 0 && 8 % a0.Hkv == 0) {
        // c + 1 <= kResidentRanges * W  <=>  q_start + r < kResidentRanges * W * B
        const int64_t lim = (int64_t)kResidentRanges * a0.resident_blocks * a0.B - a0.q_start;
        n_res = lim < 0 ? 0 : (lim < a0.rows ? lim : a0.rows);
    }
    if (n_res > 0) {
        AttnArgs a = a0;
        a.rows = (int32_t)n_res;
        hipError_t e = launch_prefill_resident<D>(a, stream);
        if (e == hipErrorNotSupported)
            n_res = 0;  // the sliced launches take every row
        else if (e != hipSuccess)
            return e;
    }
    if (n_res == a0.rows)
        return hipSuccess;
    AttnArgs a = a0;
    const int64_t r0 = n_res;
    a.rows = (int32_t)(a0.rows - r0);
    a.q_start = a0.q_start + r0;
    a.q = a0.q + r0 * a0.Hq * D;
    a.gate = a0.gate + r0 * a0.Hq;
    a.idx = a0.idx + r0 * a0.k;
    a.out = a0.out + r0 * a0.Hq * D;
    a.lse = a0.lse ? a0.lse + r0 * a0.Hq : nullptr;
    return launch_prefill_sliced<D>(a, stream);
}

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t stream)
{
    if (a.rows <= 0)
        return hipSuccess;
    if (!a.q || !a.out || (!a.idx && !a.window))
        return hipErrorInvalidValue;  // never launch without the tensors the kernels touch
    if (a.slice_blocks > 0) {
        switch (a.d) {
        case 64: return launch_prefill_ws<64>(a, stream);
        case 128: return launch_prefill_ws<128>(a, stream);
        case 192: return launch_prefill_ws<192>(a, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.d) {
    case 64: return launch_prefill_d<64>(a, stream);
    case 128: return launch_prefill_d<128>(a, stream);
    case 192: return launch_prefill_d<192>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

int prefill_state_stride(int d)
{
    return 4 * (d / 16) + 4;
}

hipError_t launch_swa(const AttnArgs &a, hipStream_t stream)
{
    if (a.rows <= 0)
        return hipSuccess;
    if (!a.q || !a.out || (!a.idx && !a.window))
        return hipErrorInvalidValue;  // never launch without the tensors the kernels touch
    switch (a.d) {
    case 64: return launch_swa_d<64>(a, stream);
    case 128: return launch_swa_d<128>(a, stream);
    case 192: return launch_swa_d<192>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream)
{
    if (a.rows <= 0)
        return hipSuccess;
    if (!a.q || !a.out || (!a.idx && !a.window))
        return hipErrorInvalidValue;  // never launch without the tensors the kernels touch
    switch (a.d) {
    case 64: return launch_decode_d<64>(a, stream);
    case 128: return launch_decode_d<128>(a, stream);
    case 192: return launch_decode_d<192>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// ============================================================================ backward
// Backward of the gated sparse attention with the selection fixed (the pages name training
// at long context among the costs of full attention; ai.info "Sparse GQA targets
// million-token context").  With P_s = exp(z_s - lse) the forward's probabilities,
// a = sum_s P_s v_s, out = sigmoid(G) a and g_out = dL/dout:
//   D = g_out . out (= da . a),  dG = D (1 - sigmoid(G)),  da = sigmoid(G) g_out,
//   dP_s = da . v_s,  dz_s = P_s (dP_s - D),
//   dq = scale sum_s dz_s k_s,  dk_s = scale sum_(t,h) dz_s q,  dv_s = sum_(t,h) P_s da.
// Without the forward output, D is formed as sum_s P_s dP_s from the kernel's own fp32 P and
// dP (a first sweep over the row): then the dz of a row sum to zero and each dz carries only
// its own bf16 rounding, instead of an error of D shared by every attended key.  Given the
// bf16 forward output, D = g_out . out is one elementwise pass and k_bwd_dq makes one sweep:
// half the dq gathers, at the price of that shared error (one bf16 rounding of out per term).
// Launches: k_bwd_prep (da), a zero fill and k_bwd_bitmap (for every key block the set of
// query rows that selected it, one bit per row, by atomicOr, whose result does not depend on
// order), k_bwd_dq (query-major, the forward's wave: a sweep for D and dG, then a second with
// dP^T = V da^T and K staged for dq^T += K^T dz^T), and k_bwd_dkdv (key-major: a wave per
// 16-token tile of a block and KV group, walking the tile's query rows in a fixed order, so dK
// and dV are sums in a fixed order and written once).
__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 pack4_bf16(float x0, float x1, float x2, float x3)
{
    const uint64_t w = (uint64_t)pack_bf16x2(x0, x1) | ((uint64_t)pack_bf16x2(x2, x3) << 32);
    return __builtin_bit_cast(s16x4, w);
}

constexpr float kLog2e = 1.4426950408889634f;

// One wave per (row, head), the waves striding over all of them (the grid is capped, so the
// launch stays inside 32-bit work-item counts at any T): da = sigmoid(G) g_out, rounded to
// bf16 for the matrix cores.  Given the forward output, also D = g_out . out (fp32 products,
// lane partial sums added by a fixed butterfly) and dG = D (1 - sigmoid(G)).
__global__ __launch_bounds__(256) void k_bwd_prep(BwdArgs a)
{
    const int64_t nrow = (int64_t)a.rows * a.Hq;
    const int lane = threadIdx.x & 63;
    const int d = a.d;
    if (!a.out && d % 8 == 0 && ((uintptr_t)a.dout & 15u) == 0) {
        // dA alone from a 16-byte aligned dout: a thread per 8 consecutive elements (16 bytes,
        // all of one row), the rows as one flat array (2 bytes per lane took 3.0 ms for the 128K
        // backward's 6.4 GB); dA sits at the start of the 256-byte aligned workspace
        const int64_t n8 = nrow * (d / 8);
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
             i += (int64_t)gridDim.x * blockDim.x) {
            const int64_t row = i / (d / 8);
            const float sg = sigmoid_f32(bf16_bits_to_f32(a.gate[row]));
            const u32x4 g = load16_stream(a.dout + i * 8);
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                o[w] = pack_bf16x2(sg * bf16_bits_to_f32(g[w] & 0xffffu),
                                   sg * bf16_bits_to_f32(g[w] >> 16));
            *reinterpret_cast<u32x4 *>(a.da + i * 8) = o;
        }
        return;
    }
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < nrow;
         row += (int64_t)gridDim.x * 4) {
        const uint16_t *go = a.dout + row * d;
        const float sg = sigmoid_f32(bf16_bits_to_f32(a.gate[row]));
        float part = 0.f;
        for (int e = lane; e < d; e += 64) {
            const float g = bf16_bits_to_f32(go[e]);
            a.da[row * d + e] = (uint16_t)f32_to_bf16_bits(sg * g);
            if (a.out)
                part = fmaf(g, bf16_bits_to_f32(a.out[row * d + e]), part);
        }
        if (a.out) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                part += __shfl_xor(part, o);
            if (lane == 0) {
                a.dsum[row] = part;
                a.dgate[row] = part * (1.0f - sg);
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_bwd_zero(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

// One thread per selection entry (grid-stride, capped grid): set bit r of block j's row.
__global__ __launch_bounds__(256) void k_bwd_bitmap(BwdArgs a)
{
    const int64_t n = (int64_t)a.rows * a.k;
    for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < n;
         gid += (int64_t)gridDim.x * 256) {
        const int64_t r = gid / a.k;
        const int32_t j = a.idx[gid];
        const int64_t c = (a.q_start + r) / a.B;
        if (j < 0 || (int64_t)j > c || (int64_t)j >= a.nblk)
            continue;
        atomicOr(&a.bits[(int64_t)j * a.bits_ld + (r >> 5)], 1u << (r & 31));
    }
}

// The dq sweeps gather a step's K rows whole (16-byte piece f = lane + 64 ci is piece
// f % (D/8) of slot f / (D/8), so each load instruction reads whole rows), place them in the
// wave's buffer [slot][D + 8] and only then request the step's V rows in the A-operand layout:
// with both in flight at once the kernel had no registers left for whole-row K (it spilled),
// and whole-row K reads made the backward 733 -> 685 ms at 128K.
template <int D>
__device__ __forceinline__ void stage_k_whole(const uint16_t *__restrict__ Kg, int64_t row_elems,
                                              int s_lo, int s_hi, uint16_t *buf)
{
    const int lane = threadIdx.x & 63;
    u32x4 kp[D / 16];
#pragma unroll
    for (int ci = 0; ci < D / 16; ++ci) {
        const int f = lane + 64 * ci;
        const int slot = f / (D / 8), piece = f - slot * (D / 8);
        const int64_t sk = ((int64_t)(uint32_t)__shfl(s_lo, slot)) |
                           ((int64_t)__shfl(s_hi, slot) << 32);
        kp[ci] = load16(Kg + sk * row_elems + piece * 8);
    }
    wave_lds_handoff();
#pragma unroll
    for (int ci = 0; ci < D / 16; ++ci) {
        const int f = lane + 64 * ci;
        const int slot = f / (D / 8), piece = f - slot * (D / 8);
        uint2 *dst = reinterpret_cast<uint2 *>(buf + slot * (D + 8) + piece * 8);
        dst[0] = uint2{kp[ci][0], kp[ci][1]};
        dst[1] = uint2{kp[ci][2], kp[ci][3]};
    }
    wave_lds_handoff();
}

// V rows of the step's slots 16 h + col in the MFMA A-operand layout (dims 32 kk + 8 q4).
template <int D>
__device__ __forceinline__ void v_operand_loads(const uint16_t *__restrict__ Vg, int64_t row_elems,
                                                int s_lo, int s_hi, u32x4 (&vv)[2][D / 32])
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int sl = h * 16 + col;
        const int64_t sv = ((int64_t)(uint32_t)__shfl(s_lo, sl)) |
                           ((int64_t)__shfl(s_hi, sl) << 32);
        const uint16_t *vr = Vg + sv * row_elems + q4 * 8;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            vv[h][kk] = load16(vr + kk * 32);
    }
}

// S^T = K Q^T from the staged K rows and dP^T = V dA^T from the V rows in registers; lane
// holds slots 16 h + 4 q4 + r of head col.
template <int D>
__device__ __forceinline__ void sdp_products(const uint16_t *buf, const u32x4 (&vv)[2][D / 32],
                                             const bf16x8 (&qf)[D / 32],
                                             const bf16x8 (&daf)[D / 32], f32x4 (&sc)[2],
                                             f32x4 (&dp)[2])
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        sc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const u32x4 ka =
                *reinterpret_cast<const u32x4 *>(buf + (h * 16 + col) * (D + 8) + kk * 32 + q4 * 8);
            sc[h] = mfma_16x16x32(as_bf16x8(ka), qf[kk], sc[h]);
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        dp[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            dp[h] = mfma_16x16x32(as_bf16x8(vv[h][kk]), daf[kk], dp[h]);
    }
}

// First sweep of a wave's (row, group): D = sum_s P_s dP_s per head (this lane's share, added
// to `part`), from the same fp32 P and dP the second sweep uses, so the dz of a row sum to
// zero.
template <int D>
__device__ __forceinline__ float dsum_range(const uint16_t *__restrict__ Kg,
                                            const uint16_t *__restrict__ Vg, int Hkv,
                                            const SparseTokens &src, const bf16x8 (&qf)[D / 32],
                                            const bf16x8 (&daf)[D / 32], float scale_log2,
                                            float lse2, uint16_t *vs, float part = 0.f)
{
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int64_t row_elems = (int64_t)Hkv * D;
    const int nsteps = src.steps();
    int wbase = -(1 << 30);
    for (int step = 0; step < nsteps; ++step) {
        int64_t s_ld;
        bool valid;
        src.slot(step, lane & 31, wbase, s_ld, valid);
        const uint64_t vmask = __ballot(valid);
        const int s_lo = (int)(s_ld & 0xffffffff), s_hi = (int)(s_ld >> 32);
        stage_k_whole<D>(Kg, row_elems, s_lo, s_hi, vs);
        u32x4 vv[2][D / 32];
        v_operand_loads<D>(Vg, row_elems, s_lo, s_hi, vv);
        f32x4 sc[2], dp[2];
        sdp_products<D>(vs, vv, qf, daf, sc, dp);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = h * 16 + q4 * 4 + r;
                if ((vmask >> slot) & 1ull)
                    part += fast_exp2(sc[h][r] * scale_log2 - lse2) * dp[h][r];
            }
    }
    return part;
}

// dq of one wave's (row, group) over its selected tokens; acc = dq^T (unscaled).  The staged
// K rows serve S^T and then dq^T += K^T dz^T, read transposed.
template <int D>
__device__ __forceinline__ void dq_range(const uint16_t *__restrict__ Kg,
                                         const uint16_t *__restrict__ Vg, int Hkv,
                                         const SparseTokens &src, const bf16x8 (&qf)[D / 32],
                                         const bf16x8 (&daf)[D / 32], float scale_log2,
                                         float lse2, float dsum, uint16_t *ks,
                                         f32x4 (&acc)[D / 16])
{
    constexpr int kLd = D + 8;
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int64_t row_elems = (int64_t)Hkv * D;
    const int nsteps = src.steps();
    int wbase = -(1 << 30);
    for (int step = 0; step < nsteps; ++step) {
        int64_t s_ld;
        bool valid;
        src.slot(step, lane & 31, wbase, s_ld, valid);
        const uint64_t vmask = __ballot(valid);
        const int s_lo = (int)(s_ld & 0xffffffff), s_hi = (int)(s_ld >> 32);
        stage_k_whole<D>(Kg, row_elems, s_lo, s_hi, ks);
        u32x4 vv[2][D / 32];
        v_operand_loads<D>(Vg, row_elems, s_lo, s_hi, vv);
        f32x4 sc[2], dp[2];
        sdp_products<D>(ks, vv, qf, daf, sc, dp);
        float dz[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = h * 16 + q4 * 4 + r;
                const bool ok = (vmask >> slot) & 1ull;
                const float p = ok ? fast_exp2(sc[h][r] * scale_log2 - lse2) : 0.f;
                dz[h][r] = p * (dp[h][r] - dsum);
            }
        u32x4 zw;
        zw[0] = pack_bf16x2(dz[0][0], dz[0][1]);
        zw[1] = pack_bf16x2(dz[0][2], dz[0][3]);
        zw[2] = pack_bf16x2(dz[1][0], dz[1][1]);
        zw[3] = pack_bf16x2(dz[1][2], dz[1][3]);
        const bf16x8 zf = as_bf16x8(zw);
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
            acc[mt] = mfma_16x16x32(vt_fragment(ks, kLd, mt * 16), zf, acc[mt]);
    }
}

template <int D, bool kGroupPerXcd>
__global__ __launch_bounds__(512) void k_bwd_dq(BwdArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    const int wave = wave_index(), lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const int hpg = a.Hq / a.Hkv;
    int64_t r;
    int g;
    if (!wave_row_group<kGroupPerXcd>(a, r, g))
        return;
    const int64_t t = a.q_start + r;
    const int64_t c = t / a.B;
    const int nvalid = (int)((c + 1 < a.k) ? c + 1 : a.k);
    const int64_t head0 = r * a.Hq + (int64_t)g * hpg;
    bf16x8 qf[D / 32], daf[D / 32];
    load_q<D>(a.q + head0 * D, hpg, qf);
    load_q<D>(a.da + head0 * D, hpg, daf);
    const float lse2 = col < hpg ? a.lse[head0 + col] * kLog2e : 0.f;
    const SparseTokens src{a.idx + r * a.k, 0, nvalid, t, c, a.B, entry_window<D>(lds)};
    uint16_t *vs = lds + wave * attn_vbuf_elems(D);
    float dsum;
    if (a.out) {
        // D = g_out . out, formed by k_bwd_prep
        dsum = col < hpg ? a.dsum[head0 + col] : 0.f;
    } else {
        // D = sum_s P_s dP_s (so that dG = D (1 - sigmoid(G)) and the dz of the row sum to 0)
        dsum = sum_across_rows(dsum_range<D>(a.kc + (int64_t)g * D, a.vc + (int64_t)g * D,
                                             a.Hkv, src, qf, daf, a.scale_log2, lse2, vs));
        if (col < hpg && q4 == 0) {
            a.dsum[head0 + col] = dsum;
            a.dgate[head0 + col] =
                dsum * (1.0f - sigmoid_f32(bf16_bits_to_f32(a.gate[head0 + col])));
        }
    }
    f32x4 acc[D / 16];
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dq_range<D>(a.kc + (int64_t)g * D, a.vc + (int64_t)g * D, a.Hkv, src, qf, daf, a.scale_log2,
                lse2, dsum, vs, acc);
    if (col < hpg) {
        float *dst = a.dq + (head0 + col) * D + q4 * 4;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
            *reinterpret_cast<f32x4 *>(dst + mt * 16) = acc[mt] * a.scale;
    }
}

// dq on the resident prefill's schedule: the same persistent grid, XCD-to-group mapping,
// batches of rows (longest history first) and block ranges of width W with the same bounded
// waits, so an XCD's L2 holds about one range of its group's K/V rows while its waves sweep
// it.  The first sweep (D, when `out` is NULL) runs over all ranges of the batch, then the
// second (dz and dq), each range's entries in the same steps as a sliced launch would take
// them; D is summed per lane across the ranges in entry order.  a.prog: one progress word per
// wave (8 XCDs x 4 a.res_wgs, zero at launch), counting the ranges the wave has finished.
template <int D>
__global__ __launch_bounds__(512) void k_bwd_dq_resident(BwdArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    const int wave = wave_index(), lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const int hpg = a.Hq / a.Hkv;
    const int R = 8 / a.Hkv;                 // XCDs per KV group
    const int x = blockIdx.x & 7;            // this workgroup's XCD
    const int g = x / R, h = x % R;
    const int nw_x = a.res_wgs * 4;          // waves per XCD
    const int lw = (int)(blockIdx.x >> 3) * 4 + wave;
    const int64_t W = a.res_w;
    uint32_t *prog = a.prog + (int64_t)x * nw_x;
    const int64_t per_batch = (int64_t)R * nw_x;
    const uint16_t *Kg = a.kc + (int64_t)g * D, *Vg = a.vc + (int64_t)g * D;
    uint16_t *vs = lds + wave * attn_vbuf_elems(D);
    uint32_t done = 0;                       // ranges finished in the earlier batches and sweeps
    for (int64_t b = 0; b * per_batch < a.rows; ++b) {
        const uint32_t done_batch0 = done;   // the batch's first sweep starts without a wait
        const int64_t j0 = b * per_batch + (int64_t)h * nw_x;
        const int64_t left = (int64_t)a.rows - j0;
        const int nval = (int)(left < 0 ? 0 : (left < nw_x ? left : nw_x));
        const int64_t c_max = (a.q_start + (int64_t)a.rows - 1 - b * per_batch) / a.B;
        const int S = (int)(c_max / W) + 1;
        const bool live = lw < nval;
        const int64_t r = uni((int64_t)a.rows - 1 - (j0 + lw));
        const int64_t t = a.q_start + r;
        const int64_t c = uni(live ? t / a.B : (int64_t)0);
        const int nvalid = (int)((c + 1 < a.k) ? c + 1 : a.k);
        const int last = uni((int)(c / W));
        const bool sliced = c >= 2 * (int64_t)a.k;
        const int32_t *row = a.idx + (live ? r : 0) * a.k;
        const int first_slice = uni(live && sliced ? (int)((int64_t)row[0] / W) : last);
        const int64_t head0 = (live ? r : 0) * a.Hq + (int64_t)g * hpg;
        const float lse2 = live && col < hpg ? a.lse[head0 + col] * kLog2e : 0.f;
        // one sweep over the batch's ranges: body(src) for this row's entries of each range
        auto sweep = [&](auto body) {
            int e_lo = 0;
            for (int s = 0; s < S; ++s) {
                // most of the XCD's waves of this batch are done with the previous range
                if ((s > 0 || done != done_batch0) && nval > 0)
                    resident_wait(prog, nw_x, done + (uint32_t)s, nval - nval / kResidentSlack);
                if (live && s >= first_slice && s <= last) {
                    const int e_hi =
                        uni(s == last ? nvalid : entries_below(row, nvalid, (int64_t)(s + 1) * W));
                    if (e_hi > e_lo)
                        body(SparseTokens{row, e_lo, e_hi, t, c, a.B, entry_window<D>(lds)});
                    e_lo = e_hi;
                }
                if (live && lane == 0)
                    __hip_atomic_store(prog + lw, done + (uint32_t)s + 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            done += (uint32_t)S;
        };
        float dsum;
        if (a.out) {
            dsum = live && col < hpg ? a.dsum[head0 + col] : 0.f;  // k_bwd_prep's D
        } else {
            float part = 0.f;
            sweep([&](const SparseTokens &src) {
                bf16x8 qf[D / 32], daf[D / 32];
                load_q<D>(a.q + head0 * D, hpg, qf);
                load_q<D>(a.da + head0 * D, hpg, daf);
                part = dsum_range<D>(Kg, Vg, a.Hkv, src, qf, daf, a.scale_log2, lse2, vs, part);
            });
            dsum = sum_across_rows(part);
            if (live && col < hpg && q4 == 0) {
                a.dsum[head0 + col] = dsum;
                a.dgate[head0 + col] =
                    dsum * (1.0f - sigmoid_f32(bf16_bits_to_f32(a.gate[head0 + col])));
            }
        }
        f32x4 acc[D / 16];
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
            acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        sweep([&](const SparseTokens &src) {
            bf16x8 qf[D / 32], daf[D / 32];
            load_q<D>(a.q + head0 * D, hpg, qf);
            load_q<D>(a.da + head0 * D, hpg, daf);
            dq_range<D>(Kg, Vg, a.Hkv, src, qf, daf, a.scale_log2, lse2, dsum, vs, acc);
        });
        if (live && col < hpg) {
            float *dst = a.dq + (head0 + col) * D + q4 * 4;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
                *reinterpret_cast<f32x4 *>(dst + mt * 16) = acc[mt] * a.scale;
        }
    }
}

// dK and dV of one 16-token tile of a key block for one KV group (one wave), over the query
// rows whose selection holds the block.  Per row: S = q K^T and dP = dA V^T with M = heads, so
// each lane holds heads 4 q4 + i of token col - exactly the A operand of the 16x16x16
// products dV += P^T dA and dK += dz^T q (M = tokens, K = heads); q and dA sit in LDS, where
// the B operands are read.  A wave walks its rows from the last one down (the order of every
// dK / dV sum), and the next row's q and dA are loaded while the current one is computed.
// Two schedules share these pieces: k_bwd_dkdv (one launch per slice of rows, the sums carried
// from slice to slice through the fp32 outputs) and k_bwd_dkdv_resident (a persistent grid
// whose waves keep their tile's sums in registers while the waves of an XCD sweep the rows
// together in phases).

// A wave's tile: its tokens, its group's K and V rows of those tokens as B operands (token col;
// padding lanes repeat token s0), the byte offsets of its staged q / dA pieces, and its LDS.
template <int D>
struct DkdvTile {
    int64_t s0;  // first token of the tile
    int ntok;    // tokens of the tile (<= 0: a tile past the end of a short last block)
    int g, hpg;
    bf16x8 kB[D / 32], vB[D / 32];
    uint32_t poff[D / 32];
    uint16_t *qs, *ds;  // staged q and dA rows [16][D + 8]
};

template <int D>
__device__ __forceinline__ void dkdv_tile(const BwdArgs &a, int64_t j, int tile, int g,
                                          uint16_t *lds_wave, DkdvTile<D> &c)
{
    constexpr int kLd = D + 8;
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    c.g = g;
    c.hpg = a.Hq / a.Hkv;
    c.s0 = j * a.B + (int64_t)tile * 16;
    int64_t ntok = a.B - tile * 16;
    ntok = ntok < 16 ? ntok : 16;
    ntok = a.L - c.s0 < ntok ? a.L - c.s0 : ntok;
    c.ntok = (int)ntok;
    c.qs = lds_wave;
    c.ds = lds_wave + 16 * kLd;
    const int64_t row_elems = (int64_t)a.Hkv * D;
    // (a tile past the end of a short last block reads the last token; it is never used)
    const int64_t sc_tok = col < ntok ? c.s0 + col : (ntok > 0 ? c.s0 : a.L - 1);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        c.kB[kk] = as_bf16x8(load16(a.kc + sc_tok * row_elems + (int64_t)g * D + kk * 32 + q4 * 8));
        c.vB[kk] = as_bf16x8(load16(a.vc + sc_tok * row_elems + (int64_t)g * D + kk * 32 + q4 * 8));
    }
    // whole rows: 16-byte piece f = lane + 64 kk of the 16 staged rows is piece f % (D/8) of
    // row f / (D/8); the group's heads are contiguous, so each load instruction reads whole
    // rows (rows past the group's heads repeat its last head, whose P and dz are masked to
    // zero).  The byte offsets within the group's rows are the same for every query row.
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const int f = lane + 64 * kk;
        const int hd = f / (D / 8), pc = f - hd * (D / 8);
        c.poff[kk] = (uint32_t)(((hd < c.hpg ? hd : c.hpg - 1) * D + pc * 8) * 2);
    }
}

// q and dA of the group's heads of row r, lse / D of head col (natural log; they reach the
// lanes holding heads 4 q4 + i by shuffles where they are used).  The loads are unconditional,
// so none of them makes the wave wait before the values are used.
template <int D>
__device__ __forceinline__ void dkdv_fetch(const BwdArgs &a, const DkdvTile<D> &c, int64_t r,
                                           u32x4 (&qa)[D / 32], u32x4 (&da)[D / 32], float &l1,
                                           float &ds1)
{
    const int col = threadIdx.x & 15;
    const int64_t h0 = r * a.Hq + (int64_t)c.g * c.hpg;  // the group's first head of row r
    const char *qb = reinterpret_cast<const char *>(a.q + h0 * D);
    const char *db = reinterpret_cast<const char *>(a.da + h0 * D);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        qa[kk] = load16(qb + c.poff[kk]);
        da[kk] = load16(db + c.poff[kk]);
    }
    const int64_t hr = h0 + (col < c.hpg ? col : c.hpg - 1);
    l1 = a.lse[hr];
    ds1 = a.dsum[hr];
}

template <int D>
__device__ __forceinline__ void dkdv_stage(const DkdvTile<D> &c, const u32x4 (&qa)[D / 32],
                                           const u32x4 (&da)[D / 32])
{
    constexpr int kLd = D + 8;
    const int lane = threadIdx.x & 63;
    wave_lds_handoff();
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const int f = lane + 64 * kk;
        const int hd = f / (D / 8), pc = f - hd * (D / 8);
        uint2 *dq_ = reinterpret_cast<uint2 *>(c.qs + hd * kLd + pc * 8);
        uint2 *dd_ = reinterpret_cast<uint2 *>(c.ds + hd * kLd + pc * 8);
        dq_[0] = uint2{qa[kk][0], qa[kk][1]};
        dq_[1] = uint2{qa[kk][2], qa[kk][3]};
        dd_[0] = uint2{da[kk][0], da[kk][1]};
        dd_[1] = uint2{da[kk][2], da[kk][3]};
    }
    wave_lds_handoff();
}

// The products of the staged row r (lse1 / ds1: its lse and D of head col) added to dk / dv.
template <int D>
__device__ __forceinline__ void dkdv_products(const BwdArgs &a, const DkdvTile<D> &c, int64_t r,
                                              float lse1, float ds1, f32x4 (&dk)[D / 16],
                                              f32x4 (&dv)[D / 16])
{
    constexpr int kLd = D + 8;
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const int64_t t = a.q_start + r;
    // S = q K^T and dP = dA V^T from the staged rows
    f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const u32x4 qa = *reinterpret_cast<const u32x4 *>(c.qs + col * kLd + kk * 32 + q4 * 8);
        const u32x4 da = *reinterpret_cast<const u32x4 *>(c.ds + col * kLd + kk * 32 + q4 * 8);
        sc = mfma_16x16x32(as_bf16x8(qa), c.kB[kk], sc);
        dp = mfma_16x16x32(as_bf16x8(da), c.vB[kk], dp);
    }
    // lane holds heads 4 q4 + i of token col
    float p[4], dz[4];
    const bool tok_ok = col < c.ntok && c.s0 + col <= t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = tok_ok && q4 * 4 + i < c.hpg;
        const float lse_i = __shfl(lse1, q4 * 4 + i), ds_i = __shfl(ds1, q4 * 4 + i);
        p[i] = ok ? fast_exp2(sc[i] * a.scale_log2 - lse_i * kLog2e) : 0.f;
        dz[i] = p[i] * (dp[i] - ds_i) * a.scale;
    }
    const s16x4 pa = pack4_bf16(p[0], p[1], p[2], p[3]);
    const s16x4 za = pack4_bf16(dz[0], dz[1], dz[2], dz[3]);
    // B[k = head 4 q4 + i][n = dim 16 nt + col] of dA and q, read transposed
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
        dv[nt] = mfma_16x16x16(pa, tr_quad(c.ds, kLd, nt * 16), dv[nt]);
        dk[nt] = mfma_16x16x16(za, tr_quad(c.qs, kLd, nt * 16), dk[nt]);
    }
}

// The rows of one block's bitmap row in words [w0, top], last first.  The words are read 64 at
// a time (lane l: word top - l) and the wave finds the non-zero ones by ballot, so finding the
// next row costs no dependent load.  Uniform across the wave.
struct RowWalk {
    const uint32_t *brow;
    int64_t w0, top, w;
    uint32_t lw, word;
    uint64_t nz;
    __device__ __forceinline__ void start(const uint32_t *row_bits, int64_t lo, int64_t hi)
    {
        const int lane = threadIdx.x & 63;
        brow = row_bits;
        w0 = lo;
        top = hi;
        lw = top - lane >= w0 ? brow[top - lane] : 0u;
        nz = __ballot(lw != 0u);
        word = 0u;
        w = top;
    }
    __device__ __forceinline__ bool next(int64_t &r)
    {
        const int lane = threadIdx.x & 63;
        while (word == 0u) {
            if (nz == 0ull) {
                top -= 64;
                if (top < w0)
                    return false;
                lw = top - lane >= w0 ? brow[top - lane] : 0u;
                nz = __ballot(lw != 0u);
                continue;
            }
            const int l = __builtin_ctzll(nz);  // the highest non-zero word left
            nz &= nz - 1ull;
            word = (uint32_t)__builtin_amdgcn_readlane((int)lw, l);
            w = top - l;
        }
        const int b = 31 - __builtin_clz(word);
        word &= ~(1u << b);
        r = (w << 5) + b;
        return true;
    }
};

// Adds the rows of `it` (the first one, r, already staged with lse1 / ds1) to dk / dv, each
// row's successor in flight while it is computed.
template <int D>
__device__ __forceinline__ void dkdv_walk(const BwdArgs &a, const DkdvTile<D> &c, RowWalk &it,
                                          int64_t r, float lse1, float ds1, f32x4 (&dk)[D / 16],
                                          f32x4 (&dv)[D / 16])
{
    bool have = true;
#pragma unroll 1
    while (have) {
        int64_t rn = 0;
        const bool have_next = it.next(rn);
        u32x4 nq[D / 32], nd[D / 32];
        float nl = 0.f, ns = 0.f;
        if (have_next)
            dkdv_fetch<D>(a, c, rn, nq, nd, nl, ns);
        dkdv_products<D>(a, c, r, lse1, ds1, dk, dv);
        if (have_next) {
            dkdv_stage<D>(c, nq, nd);
            lse1 = nl;
            ds1 = ns;
        }
        r = rn;
        have = have_next;
    }
}

// lane holds dK / dV of token 4 q4 + i, dim 16 nt + col
template <int D>
__device__ __forceinline__ void dkdv_store(const BwdArgs &a, const DkdvTile<D> &c,
                                           const f32x4 (&dk)[D / 16], const f32x4 (&dv)[D / 16])
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = q4 * 4 + i;
        if (tok < c.ntok) {
            const int64_t base = ((c.s0 + tok) * a.Hkv + c.g) * D;
#pragma unroll
            for (int nt = 0; nt < D / 16; ++nt) {
                a.dk[base + nt * 16 + col] = dk[nt][i];
                a.dv[base + nt * 16 + col] = dv[nt][i];
            }
        }
    }
}

// Sliced schedule: a workgroup takes 4 tiles of one group (group = blockIdx % Hkv, so with Hkv
// dividing 8 each XCD's L2 serves one group's rows).  One launch covers the rows
// [row_lo, row_hi) only: the launcher runs the slices from the last one down, so that the q
// and dA rows in use at any time fit in the memory-side cache, and each wave carries its sums
// over from the previous slice through the fp32 dK / dV outputs (same summation order as a
// single sweep).
template <int D>
__global__ __launch_bounds__(512) void k_bwd_dkdv(BwdArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    constexpr int kLd = D + 8;
    const int ntile = (a.B + 15) / 16;
    const int g = (int)(blockIdx.x % (unsigned)a.Hkv);
    const int wave = wave_index(), lane = threadIdx.x & 63;
    const int64_t tid = (int64_t)(blockIdx.x / (unsigned)a.Hkv) * 4 + wave;  // tile index
    if (tid >= a.nblk * ntile)
        return;
    const int64_t j = tid / ntile;
    const int tile = (int)(tid - j * ntile);
    const int col = lane & 15, q4 = lane >> 4;
    DkdvTile<D> c;
    dkdv_tile<D>(a, j, tile, g, lds + wave * 2 * 16 * kLd, c);
    if (c.ntok <= 0)
        return;  // a tile past the end of a short last block
    f32x4 dk[D / 16], dv[D / 16];

    // this launch's rows [row_lo, row_hi) (row_lo a multiple of 32); none before first_row
    // can select block j
    const int64_t first_row = j * a.B - a.q_start;
    const int64_t w_lo = a.row_lo >> 5;
    const int64_t w0 = first_row > 0 && (first_row >> 5) > w_lo ? first_row >> 5 : w_lo;
    RowWalk it;
    it.start(a.bits + j * a.bits_ld, w0, ((a.row_hi + 31) >> 5) - 1);
    int64_t r;
    if (!it.next(r))
        return;  // no row of this slice selects the block: its sums stay as they are
    float lse1, ds1;  // the staged row's lse and D of head col
    {
        u32x4 qa[D / 32], da[D / 32];
        dkdv_fetch<D>(a, c, r, qa, da, lse1, ds1);
        dkdv_stage<D>(c, qa, da);
    }
    // continue the sums of the slices already done (the launcher zeroes dK and dV first)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = q4 * 4 + i;
        const int64_t base = ((c.s0 + (tok < c.ntok ? tok : 0)) * a.Hkv + g) * D;
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) {
            dk[nt][i] = tok < c.ntok ? a.dk[base + nt * 16 + col] : 0.f;
            dv[nt][i] = tok < c.ntok ? a.dv[base + nt * 16 + col] : 0.f;
        }
    }
    // Let these loads land here: the wait the compiler would otherwise put before the first
    // product in the loop (it cannot tell they finished) would also drain each row's prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    dkdv_walk<D>(a, c, it, r, lse1, ds1, dk, dv);
    dkdv_store<D>(a, c, dk, dv);
}

// Resident schedule: a persistent grid of exactly the resident workgroups.  The waves of one
// XCD take a batch of nw_x consecutive tiles of the XCD's KV group (the R = 8 / Hkv XCDs of a
// group split the group's batch of R * nw_x tiles; batches from the last tiles down) and keep
// their sums in registers while they sweep the query rows from the last one down in phases of
// a.row_slice rows: a wave starts phase s once most waves of its XCD have finished phase s - 1,
// so the XCD's L2 holds about one phase's q and dA rows at a time.  The wait only orders the
// work for the caches (it guards no data; a wave that stops waiting at the bound computes the
// same result), and each tile's rows are added in the same order as in the sliced schedule,
// so dK and dV are the same bits.  Every tile's dK / dV is written once, so the outputs need
// no clearing.  a.prog: one progress word per wave (8 XCDs x 4 a.res_wgs, zero at launch).
template <int D>
__global__ __launch_bounds__(512) void k_bwd_dkdv_resident(BwdArgs a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    constexpr int kLd = D + 8;
    const int wave = wave_index();
    const int R = 8 / a.Hkv;                 // XCDs per KV group
    const int x = blockIdx.x & 7;            // this workgroup's XCD
    const int g = x / R, h = x % R;
    const int nw_x = a.res_wgs * 4;          // waves per XCD
    const int lw = (int)(blockIdx.x >> 3) * 4 + wave;
    uint32_t *prog = a.prog + (int64_t)x * nw_x;
    const int ntile = (a.B + 15) / 16;
    const int64_t ntiles = a.nblk * ntile;
    const int64_t per_batch = (int64_t)R * nw_x;
    const int64_t pw = a.row_slice >> 5;     // bitmap words per phase
    const int64_t wtop = ((int64_t)a.rows - 1) >> 5;
    uint16_t *lds_wave = lds + wave * 2 * 16 * kLd;
    uint32_t done = 0;                       // phases of the earlier batches
    for (int64_t b = 0; b * per_batch < ntiles; ++b) {
        // this XCD's tiles of the batch, from the last one down
        const int64_t i0 = b * per_batch + (int64_t)h * nw_x;
        const int64_t left = ntiles - i0;
        const int nval = (int)(left < 0 ? 0 : (left < nw_x ? left : nw_x));
        if (nval == 0)
            break;                           // the other XCDs of the group took the last tiles
        // phases down to the first row that can select the XCD's lowest block of the batch
        const int64_t j_lo = (ntiles - 1 - (i0 + nval - 1)) / ntile;
        const int64_t r_lo = j_lo * a.B - a.q_start;
        const int64_t w_lo = r_lo > 0 ? r_lo >> 5 : 0;
        const int S = w_lo > wtop ? 0 : (int)((wtop - w_lo) / pw) + 1;
        const bool live = lw < nval;
        const int64_t tid = uni(live ? ntiles - 1 - (i0 + lw) : (int64_t)0);
        const int64_t j = tid / ntile;
        const int tile = (int)(tid - j * ntile);
        DkdvTile<D> c;
        dkdv_tile<D>(a, j, tile, g, lds_wave, c);
        const bool work = live && c.ntok > 0;
        f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt)
            dk[nt] = dv[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t first_row = j * a.B - a.q_start;  // none before it selects block j
        const int64_t wf = first_row > 0 ? first_row >> 5 : 0;
        const uint32_t *brow = a.bits + j * a.bits_ld;
        for (int s = 0; s < S; ++s) {
            // most of the XCD's waves of this batch are done with phase s - 1
            if (s > 0)
                resident_wait(prog, nw_x, done + (uint32_t)s, nval - nval / kResidentSlack);
            const int64_t top = wtop - (int64_t)s * pw;
            if (work && top >= wf) {
                const int64_t bot = top - pw + 1;
                RowWalk it;
                it.start(brow, bot > wf ? bot : wf, top);
                int64_t r;
                if (it.next(r)) {
                    float lse1, ds1;
                    u32x4 qa[D / 32], da[D / 32];
                    dkdv_fetch<D>(a, c, r, qa, da, lse1, ds1);
                    dkdv_stage<D>(c, qa, da);
                    dkdv_walk<D>(a, c, it, r, lse1, ds1, dk, dv);
                }
            }
            if (live && (threadIdx.x & 63) == 0)
                __hip_atomic_store(prog + lw, done + (uint32_t)s + 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (work)
            dkdv_store<D>(a, c, dk, dv);
        done += (uint32_t)S;
    }
}

// Backward workspace: dA (bf16), D (fp32), the row bitmap, then the resident dq's progress
// words, each part 256-byte aligned.
size_t attn_backward_workspace(int64_t T, int Hq, int d, int64_t nblk)
{
    const int64_t bits_ld = (((T + 31) / 32) + 3) / 4 * 4;
    const size_t da = ((size_t)T * Hq * d * 2 + 255) / 256 * 256;
    const size_t ds = ((size_t)T * Hq * 4 + 255) / 256 * 256;
    const size_t bits = ((size_t)nblk * bits_ld * 4 + 255) / 256 * 256;
    return da + ds + bits + kResidentProgressBytes;
}

// Query rows per dK / dV launch: a multiple of 32 (one bitmap word) whose q and dA take about
// 192 MiB, inside the 256 MiB memory-side cache (at 64 heads of 192: 4096 rows; 512 to 8192
// rows measured within 5 % of it at 128K, one pass over all rows 9 % slower).
static int64_t bwd_row_slice(int Hq, int d)
{
    const int64_t per_row = (int64_t)Hq * d * 2 * 2;
    const int64_t rows = ((int64_t)192 << 20) / per_row / 32 * 32;
    return rows > 32 ? rows : 32;
}

// Query rows per phase of the resident dK / dV when the caller leaves it open.  128K prefill,
// dK / dV pass (sliced: 390 ms, 17.6 % L2 hits): phases of 512 / 1024 / 2048 / 4096 rows
// 387 / 372 / 368 / 381 ms at 63 / 50 / 36 / 26 % L2 hits - the pass waits on each row's
// q / dA request about as long whether it hits the L2 or not
constexpr int64_t kDkdvPhaseRows = 2048;

// The resident dK / dV when the KV groups divide the 8 XCDs and the workspace holds the
// progress words; hipErrorNotSupported otherwise.  a.row_slice > 0 sets the phase height.
template <int D>
static hipError_t launch_bwd_dkdv_resident(const BwdArgs &a0, hipStream_t stream)
{
    if (!a0.prog || 8 % a0.Hkv != 0)
        return hipErrorNotSupported;
    const size_t lds = (size_t)4 * 2 * 16 * (D + 8) * sizeof(uint16_t);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_bwd_dkdv_resident<D>, 256,
                                                         lds);
    if (e != hipSuccess)
        return e;
    const int per_xcd = per_cu * (cus / 8);
    const int words = 8 * per_xcd * 4;  // one progress word per wave
    if (per_xcd < 1 || (size_t)words * sizeof(uint32_t) > kResidentProgressBytes)
        return hipErrorNotSupported;
    BwdArgs a = a0;
    a.res_wgs = per_xcd;
    a.row_slice = a0.row_slice > 0 ? a0.row_slice : kDkdvPhaseRows;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       a.prog, words);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_bwd_dkdv_resident<D>, dim3((unsigned)(8 * per_xcd)), dim3(256), lds,
                       stream, a);
    return hipGetLastError();
}

// The resident dq when the KV groups divide the 8 XCDs and every row's history lies within
// kResidentRanges ranges of a.res_w blocks; hipErrorNotSupported otherwise.
template <int D>
static hipError_t launch_bwd_dq_resident(const BwdArgs &a0, hipStream_t stream)
{
    if (!a0.prog || a0.res_w < 1 || 8 % a0.Hkv != 0 ||
        (a0.q_start + (int64_t)a0.rows - 1) / a0.B >= (int64_t)kResidentRanges * a0.res_w)
        return hipErrorNotSupported;
    const size_t lds = (size_t)4 * attn_wave_lds(D);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_bwd_dq_resident<D>, 256, lds);
    if (e != hipSuccess)
        return e;
    const int per_xcd = per_cu * (cus / 8);
    const int words = 8 * per_xcd * 4;  // one progress word per wave
    if (per_xcd < 1 || (size_t)words * sizeof(uint32_t) > kResidentProgressBytes)
        return hipErrorNotSupported;
    BwdArgs a = a0;
    a.res_wgs = per_xcd;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       a.prog, words);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_bwd_dq_resident<D>, dim3((unsigned)(8 * per_xcd)), dim3(256), lds, stream,
                       a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_backward_d(const BwdArgs &a, hipStream_t stream)
{
    // dq: the resident schedule where it applies, else the forward's one-pass launch shape
    hipError_t e = launch_bwd_dq_resident<D>(a, stream);
    if (e == hipErrorNotSupported) {
        if (8 % a.Hkv == 0) {
            const int R = 8 / a.Hkv;
            const int64_t ntiles = ((int64_t)a.rows + 3) / 4;
            const int64_t nwg = (ntiles + R - 1) / R * 8;
            const size_t lds = (size_t)4 * attn_wave_lds(D);
            hipLaunchKernelGGL((k_bwd_dq<D, true>), dim3((unsigned)nwg), dim3(256), lds, stream,
                               a);
        } else {
            const size_t lds = (size_t)a.Hkv * attn_wave_lds(D);
            hipLaunchKernelGGL((k_bwd_dq<D, false>), dim3((unsigned)a.rows), dim3(64 * a.Hkv),
                               lds, stream, a);
        }
        e = hipGetLastError();
    }
    if (e != hipSuccess)
        return e;
    // dK / dV: the resident schedule where it applies; else zeroed, then one launch per slice of
    // rows, last slice first
    e = launch_bwd_dkdv_resident<D>(a, stream);
    if (e != hipErrorNotSupported)
        return e;
    const int64_t nkv = a.L * a.Hkv * D;
    const unsigned zg = (unsigned)(nkv < 65536 * 256 ? (nkv + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_bwd_zero, dim3(zg), dim3(256), 0, stream, (uint32_t *)a.dk, nkv);
    hipLaunchKernelGGL(k_bwd_zero, dim3(zg), dim3(256), 0, stream, (uint32_t *)a.dv, nkv);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t slice = a.row_slice > 0 ? a.row_slice : bwd_row_slice(a.Hq, D);
    const int64_t ntiles = a.nblk * ((a.B + 15) / 16);
    const int64_t nwg = (ntiles + 3) / 4 * a.Hkv;  // 4 tiles of one group per workgroup
    const size_t lds = (size_t)4 * 2 * 16 * (D + 8) * sizeof(uint16_t);
    for (int64_t lo = ((int64_t)a.rows - 1) / slice * slice; lo >= 0; lo -= slice) {
        BwdArgs s = a;
        s.row_lo = lo;
        s.row_hi = lo + slice < a.rows ? lo + slice : a.rows;
        hipLaunchKernelGGL(k_bwd_dkdv<D>, dim3((unsigned)nwg), dim3(256), lds, stream, s);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_attn_backward(const BwdArgs &a, hipStream_t stream)
{
    if (a.rows <= 0)
        return hipSuccess;
    if (!a.q || !a.dout || !a.dq || !a.dk || !a.dv || !a.dgate || !a.da || !a.dsum || !a.bits)
        return hipErrorInvalidValue;  // never launch without the tensors the kernels touch
    const int64_t nrow = (int64_t)a.rows * a.Hq;
    const int64_t prep_wg = (nrow + 3) / 4;
    hipLaunchKernelGGL(k_bwd_prep, dim3((unsigned)(prep_wg < (1 << 20) ? prep_wg : (1 << 20))),
                       dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t words = a.nblk * a.bits_ld;
    hipLaunchKernelGGL(k_bwd_zero, dim3((unsigned)(words < 65536 * 256 ? (words + 255) / 256 : 65536)),
                       dim3(256), 0, stream, a.bits, words);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t ent = (int64_t)a.rows * a.k;
    const int64_t bm_wg = (ent + 255) / 256;
    hipLaunchKernelGGL(k_bwd_bitmap, dim3((unsigned)(bm_wg < (1 << 20) ? bm_wg : (1 << 20))),
                       dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    switch (a.d) {
    case 64: return launch_backward_d<64>(a, stream);
    case 128: return launch_backward_d<128>(a, stream);
    case 192: return launch_backward_d<192>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace sgqa
