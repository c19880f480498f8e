// sgqa_launch.hpp -- internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stdint.h>

namespace sgqa {

constexpr int kMaxSeq = 64;

// Per-sequence positions passed by value in the kernel arguments.
struct SeqPositions {
    int64_t v[kMaxSeq];
};

// Block compression of one sequence: kb[j] = mean(kp[jB .. min(jB+B, L)-1]) for j in [j0, j1).
hipError_t launch_index_build(const uint16_t *kp, uint16_t *kb, int64_t L, int P, int B,
                              int64_t j0, int64_t j1, hipStream_t stream);

// Index maintenance from the keys, all sequences in one launch: for sequence s and block
// j in [j0[s], j1[s]), kb[j] = (mean of the concatenated keys of its tokens) . W, with
// wt = W transposed ([P][width]), width = Hkv * d.
struct IndexKeysArgs {
    const uint16_t *k;       // [nseq][cache_seq_stride] of [L][width]
    int64_t cache_seq_stride;
    const uint16_t *wt;      // [P][width]
    uint16_t *kb;            // [nseq][kb_seq_stride] of [nblk][P]
    int64_t kb_seq_stride;
    int width, P, B, nseq;
    SeqPositions len, j0, j1;
};
hipError_t launch_index_from_keys(const IndexKeysArgs &a, int64_t max_blocks, hipStream_t stream);

// FP8 storage of rows: codes[r][i] = e4m3(x[r][i] / scale[r]), scale[r] = max_i |x[r][i]| / 448
// (1 for a zero row), all in fp32.
hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int cols, uint8_t *codes,
                                float *scales, hipStream_t stream);

// Indexer scores for queries [t0, t0+nq) of every sequence into ws rows
// (row = s*nq + i, row stride ld floats); only blocks j < (q_start[s]+i)/B are written.
struct ScoreArgs {
    const uint16_t *qp;
    int64_t qp_seq_stride;
    const uint16_t *kb;
    int64_t kb_seq_stride;
    SeqPositions q_start;
    int32_t nseq;
    int32_t t0;
    int32_t nq;
    int32_t P;
    int32_t B;
    int64_t max_cand;  // largest candidate count over the rows of this pass
    float *ws;
    int64_t ld;
};
hipError_t launch_scores(const ScoreArgs &a, hipStream_t stream);

// Causal top-k of every row of a score pass (see sgqa_indexer_topk).
struct SelectArgs {
    const float *ws;
    int64_t ld;
    SeqPositions q_start;
    int32_t nseq;
    int32_t t0;
    int32_t nq;
    int32_t T;
    int32_t B;
    int32_t k;
    int64_t max_cand;
    int32_t *idx;
    float *sel_scores;
};
hipError_t launch_select(const SelectArgs &a, hipStream_t stream);

// Prefill top-k without a score matrix (k_fused_* in k_indexer.hip), for the queries
// [t0, t0+nq) of every sequence; row r = s*nq + i.  Workspace arrays per pass:
// samp [rows][ns] u32, thr / cnt / queue [rows] u32, cand [rows][cap] (key, block),
// queue_ctr [2] u32 (queued rows, rows taken), fb_scores [kFusedFallbackWGs][fb_ld] fp32.
struct FusedTopkArgs {
    const uint16_t *qp;
    int64_t qp_seq_stride;
    const uint16_t *kb;
    int64_t kb_seq_stride;
    SeqPositions q_start;
    int32_t nseq, t0, nq, T, P, B, k;
    int64_t max_cand;  // largest candidate count over the rows of this pass
    int32_t ns, cap;
    uint32_t *samp, *thr, *cnt, *queue, *queue_ctr;
    uint2 *cand;
    float *fb_scores;
    int64_t fb_ld;
    int32_t *idx;
    float *sel_scores;
};
bool fused_topk_supported(int64_t max_cand, int k, int P);
void fused_topk_geometry(int64_t max_cand, int &ns, int &cap);
size_t fused_topk_row_bytes(int64_t max_cand);    // per query row of a pass
size_t fused_topk_fixed_bytes(int64_t max_cand);  // counters and fallback scratch rows
hipError_t launch_fused_topk(const FusedTopkArgs &a, hipStream_t stream);

// Decode-shaped top-k (one query per sequence): score keys for every block, then one
// selection workgroup per sequence.  The workspace holds keys [nseq][keys_ld] and unit
// maxima [nseq][units_ld] (u32).
constexpr int64_t kDecodeMaxCand = 131072;
struct DecodeTopkArgs {
    const uint16_t *qp;  // query proxy of sequence s at qp + s * qp_seq_stride
    int64_t qp_seq_stride;
    const uint16_t *kb;
    int64_t kb_seq_stride;
    SeqPositions pos;    // query position per sequence
    int32_t nseq;
    int32_t P;
    int32_t B;
    int32_t k;
    uint32_t *keys;      // [nseq][keys_ld] order-preserving score keys
    int64_t keys_ld;
    uint32_t *umax;      // [nseq][units_ld] largest key of each 16-block unit
    int64_t units_ld;
    int32_t *idx;        // [nseq][k]
    float *sel_scores;   // [nseq][k] or null
    // FP8 index (instead of kb): e4m3 codes [nseq][kbs_seq_stride][P], one fp32 scale per row
    const uint8_t *kbq;
    const float *kbs;
    int64_t kbs_seq_stride;  // rows (blocks) per sequence
};
// False when the shape is outside the decode path (then the general path is used).
bool decode_topk_supported(int64_t max_cand, int k);
int64_t decode_keys_ld(int64_t max_cand);
int64_t decode_units_ld(int64_t max_cand);
size_t decode_topk_workspace(int nseq, int64_t max_cand);
hipError_t launch_decode_topk(const DecodeTopkArgs &a, hipStream_t stream);

struct AttnArgs {
    const uint16_t *q;       // [rows][Hq][d]
    const uint16_t *kc;      // K cache base of sequence 0
    const uint16_t *vc;      // V cache base of sequence 0
    int64_t cache_seq_stride;  // elements, decode only
    const uint16_t *gate;    // [rows][Hq]
    const int32_t *idx;      // [rows][k]
    int64_t q_start;         // prefill: position of row 0
    SeqPositions qpos;       // decode: query position per sequence
    int32_t rows;            // prefill: T; decode: nseq
    int32_t Hq, Hkv, d, B, k;
    float scale_log2;        // softmax_scale * log2(e)
    uint16_t *out;
    float *lse;
    // decode split-K partials
    float *part_o;           // [nseq][npart][Hq][d]
    float *part_ml;          // [nseq][npart][Hq][3]: max, bf16-weight sum, fp32-weight sum
    int32_t nsplit;          // splits of the selection entries (one wave each)
    int32_t entries_per_split;
    int32_t npart;           // partial states per (sequence, head): one per workgroup
    int64_t window;          // sliding-window attention: tokens per window
    // sliced prefill: launch `slice` covers the history blocks [slice, slice + 1) *
    // slice_blocks of every row (0: one pass), parking the per-lane softmax state
    // (state_stride floats per lane) in `state` between launches
    int64_t slice_blocks;
    int32_t long_slices;     // ranges of a history longer than 16 slice_blocks ranges
    // resident prefill (one launch, the state kept in registers across the ranges): range
    // width in blocks for rows whose history spans at most 16 such ranges (0: not used)
    int64_t resident_blocks;
    int32_t slice;
    float *state;
    int64_t state_bytes;
    int32_t state_stride;
    // FP8 caches (decode): e4m3 codes [nseq][scale_seq_stride][Hkv][d] and one fp32 scale per
    // (token, KV head) [nseq][scale_seq_stride][Hkv]; used instead of kc / vc when kq is set
    const uint8_t *kq;
    const uint8_t *vq;
    const float *ksc;
    const float *vsc;
    int64_t scale_seq_stride;  // tokens per sequence
};
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream);
hipError_t launch_swa(const AttnArgs &a, hipStream_t stream);

// Backward of the sparse attention with the selection fixed (prefill layout: T query rows at
// q_start .. q_start+T-1 over an L-token cache).
struct BwdArgs {
    const uint16_t *q, *kc, *vc, *gate, *dout;        // forward inputs and dL/dout
    const uint16_t *out;                              // forward output or null (D from P dP)
    const float *lse;                                 // forward log-sum-exp [T][Hq]
    const int32_t *idx;                               // [T][k]
    int64_t q_start;
    int32_t rows;                                     // T
    int64_t L;
    int32_t Hq, Hkv, d, B, k;
    float scale, scale_log2;
    float *dq, *dk, *dv, *dgate;                      // [T][Hq][d], [L][Hkv][d] x2, [T][Hq]
    uint16_t *da;                                     // workspace: sigmoid(gate) dL/dout, bf16
    float *dsum;                                      // workspace: sum_s P_s dP_s per (row, head)
    uint32_t *bits;                                   // workspace: [nblk][bits_ld] row bitmap
    int64_t bits_ld;
    int64_t nblk;
    int64_t row_slice;                                // rows per dK / dV launch (0: automatic)
    int64_t row_lo, row_hi;                           // dK / dV launch: rows of this slice
    uint32_t *prog;                                   // workspace: resident dq progress words
    int64_t res_w;                                    // resident dq: range width in blocks
    int32_t res_wgs;                                  // resident dq: workgroups per XCD
};
hipError_t launch_attn_backward(const BwdArgs &a, hipStream_t stream);
size_t attn_backward_workspace(int64_t T, int Hq, int d, int64_t nblk);
int prefill_state_stride(int d);

// Workspace the resident prefill needs for its progress words: one 4-byte word per resident
// wave, at most 8 workgroups of 4 waves per CU on 256 CUs.
constexpr size_t kResidentProgressBytes = size_t(256) * 8 * 4 * sizeof(uint32_t);

// Decode split-K geometry for k selected entries of B tokens.
void decode_split_plan(int k, int B, int &nsplit, int &entries_per_split);
// Partial states per (sequence, head) the decode attention writes for nsplit splits (one per
// decode workgroup).
int decode_parts(int nsplit);

// Fixed device scratch of kScratchBytes for the entry points that allocate nothing
// (sgqa_scratch.hip): the current device's copy, looked up once per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_region(void **ptr, size_t *bytes);

} // namespace sgqa
