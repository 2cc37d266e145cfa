// rda_internal.h -- declarations shared by the library's translation units
// (launchers, workspace layout).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "rda.h"

namespace rda {

constexpr int kC = RDA_CHUNK;      // tokens per chunk
constexpr int kD = RDA_HEAD_DIM;   // dk = dv

// ---------------------------------------------------------------------------
// Workspace layout of rda_prefill (all offsets 256-byte aligned):
//
//   [table]     int32 rec[max_chunks][4]   (seq, token start, valid len, chunk-in-seq)
//               int32 seq_off[num_seqs+1]  first chunk of each sequence
//               int32 num_chunks[1]
//   [factors]   per (chunk, head), kChunkHeadBytes each, chunk-major:
//                 Tb   bf16 hi/lo of T diag(b), T = (I + L)^-1, packed as the
//                      walk's MFMA A operand (rows = tokens, K dim = tokens)
//                 Am   bf16 hi/lo of A = lower(Q K^T . Gamma), same packing
//                      (for both: the slots of token tiles 0 and 1 against
//                      key block 1 are zero; the bf16 kernels neither write
//                      nor read them)
//                 G    fp32 gamma_i (64), gamma_C / gamma_i (64), gamma_C,
//                      g_i = running sum of log a (64, at float 192)
// ---------------------------------------------------------------------------
constexpr size_t kPackBytes = size_t(kC) * kC * 2 * 2;   // hi + lo bf16, 64 x 64
constexpr size_t kGBytes = 1024;
constexpr size_t kOffTb = 0;
constexpr size_t kOffA = kOffTb + kPackBytes;
constexpr size_t kOffG = kOffA + kPackBytes;
constexpr size_t kChunkHeadBytes = kOffG + kGBytes;
constexpr int kGGam = 0;     // float offsets inside G
constexpr int kGScale = 64;
constexpr int kGC = 128;
constexpr int kGLog = 192;

// Per-(chunk, head) factors of the per-channel-decay prefill (same table in
// front), each packed as the walk's bf16 hi/lo MFMA operands:
//   Tb  T diag(b)                       rows tokens, K dim tokens   16 KiB
//   Am  A                               rows tokens, K dim tokens   16 KiB
//   Kt  K . e^G                         rows tokens, K dim keys     32 KiB
//   Qt  Q . e^G                         rows tokens, K dim keys     32 KiB
//   Kh  (K . e^{G_C - G})^T             rows keys, K dim tokens     32 KiB
//   GC  e^{G_C} per key channel, fp32                               512 B
constexpr size_t kDOffTb = 0;
constexpr size_t kDOffA = kDOffTb + kPackBytes;
constexpr size_t kDOffKt = kDOffA + kPackBytes;
constexpr size_t kDOffQt = kDOffKt + 2 * kPackBytes;
constexpr size_t kDOffKh = kDOffQt + 2 * kPackBytes;
constexpr size_t kDOffGC = kDOffKh + 2 * kPackBytes;
constexpr size_t kDiagChunkHeadBytes = kDOffGC + 512;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct TableLayout {
    size_t rec_off, seq_off_off, num_off, bytes;
};

inline TableLayout table_layout(int32_t max_chunks, int32_t num_seqs) {
    TableLayout t;
    t.rec_off = 0;
    t.seq_off_off = align256(size_t(max_chunks) * 4 * sizeof(int32_t));
    t.num_off = t.seq_off_off + align256(size_t(num_seqs + 1) * sizeof(int32_t));
    t.bytes = t.num_off + 256;
    return t;
}

// ---------------------------------------------------------------------------
// launchers (each returns the hipGetLastError() of its launch)
// ---------------------------------------------------------------------------
hipError_t launch_chunk_table(const int32_t* cu, int32_t num_seqs, int32_t total_tokens,
                              int32_t max_chunks, int32_t* rec, int32_t* seq_off,
                              int32_t* num_chunks, hipStream_t stream);

hipError_t launch_decode(const void* q, const void* k, const void* v, rda_dtype dt,
                         const float* a, const float* b, int32_t batch, int32_t heads,
                         float* S, float* o, hipStream_t stream);

// Several tokens per (batch, head); o == nullptr selects the commit-only
// kernel (no outputs, stops after the accepted tokens).
// diag: a is a per-key-channel decay [batch, tokens, H, 128] instead of a
// scalar [batch, tokens, H].
hipError_t launch_decode_tokens(const void* q, const void* k, const void* v, rda_dtype dt,
                                const float* a, const float* b, int32_t batch, int32_t tokens,
                                int32_t heads, const float* S_in, float* S_out,
                                const int32_t* accept, float* o, bool diag, hipStream_t stream);

// Prologue: raw q, k, v (bf16) -> conv, activation, q/k norm, write gate;
// a, b from the gates; the conv history.  cu == nullptr: N sequences of L
// tokens each.
struct PrologueArgs {
    const uint16_t* x[3];      // raw q, k, v [T, H, 128]
    const float* w;            // [3][H][128][K]
    const uint16_t* hin;       // [N][3][K-1][H][128] or nullptr (zeros)
    uint16_t* hout;            // same shape or nullptr
    const float* beta;         // [T, H]
    const float* delta;        // [T, H] or nullptr
    const float* glog;         // [T, H]
    float floor_log, l2eps;
    const int32_t* cu;         // [N+1] or nullptr
    int32_t N, T, H, L;
    uint16_t* out[3];          // q, k, v [T, H, 128] bf16
    float* a;                  // [T, H]
    float* b;
};
hipError_t launch_prologue(const PrologueArgs& P, int32_t K, int32_t act, hipStream_t stream);

// One decode step with the prologue in front (one token per sequence):
// raw projections, conv weights and history, gates' inputs -> the state
// update and the outputs, the history moved on (hout may be hin).
struct DecodePrologueArgs {
    const uint16_t* x[3];      // raw q, k, v [B, H, 128] bf16
    const float* w;            // [3][H][128][K]
    const uint16_t* hin;       // [B][3][K-1][H][128] or nullptr (zeros)
    uint16_t* hout;            // same shape or nullptr (no history kept)
    const float* beta;         // [B, H]
    const float* delta;        // [B, H] or nullptr
    const float* glog;         // [B, H]
    float floor_log, l2eps;
    int32_t H;
    float* S;                  // [B, H, 128, 128] in/out
    float* o;                  // [B, H, 128]
};
hipError_t launch_decode_prologue(const DecodePrologueArgs& P, int32_t batch, int32_t K,
                                  int32_t act, hipStream_t stream);

// One walk job: where the state starts (identity, S0, or zero when S0 is
// null), whether v counts (zero_v: every value taken as 0, so the walk
// applies the chunks' transition alone) and where the final state goes
// (skipped when null).
struct WalkJob {
    const float* S0;
    float* S_final;
    int identity;
    int zero_v;
};

// Per-channel decay: prep + walk after the chunk table (q, k, v in dt).
hipError_t launch_prefill_diag(const void* q, const void* k, const void* v, rda_dtype dt,
                               const float* alpha, const float* b, int32_t num_seqs,
                               int32_t heads, int32_t max_chunks, const int32_t* rec,
                               const int32_t* seq_off, const int32_t* num_chunks,
                               unsigned char* factors, const float* S0, float* o,
                               float* S_final, hipStream_t stream);
// Its two stages apart (the segmented state pass runs the walk three times
// over one prep): the prep (of the first item_end (chunk, head) items, all
// when negative), and the walk with jobs, segment runs and the
// instantiation without outputs as for launch_walk_bf16.  A walk launch may
// carry a DiagSide: a chunk range for one sequence (c_hi > 0: walk chunks
// [c_lo, c_hi) only) and prep workgroups after the walk's that prep items
// [item_lo, item_hi) of the table on the CUs the walk leaves idle.
struct DiagSide {
    int c_lo, c_hi;
    int prep_blocks;        // prep workgroups (0: none)
    int item_lo, item_hi;
    const void* q;
    const void* k;
    const float* alpha;
    const float* b;
    int walk_blocks;        // set by the launcher
};
hipError_t launch_prep_diag(const void* q, const void* k, rda_dtype dt, const float* alpha,
                            const float* b, int32_t heads, int32_t max_chunks, const int32_t* rec,
                            const int32_t* num_chunks, unsigned char* factors,
                            hipStream_t stream, int32_t item_end = -1);
hipError_t launch_walk_diag(const void* v, rda_dtype dt, int32_t num_seqs, int32_t heads,
                            const int32_t* rec, const int32_t* seq_off,
                            const int32_t* num_chunks, unsigned char* factors, float* o,
                            const WalkJob* jobs, int32_t num_jobs, int32_t seg_chunks,
                            bool outputs, hipStream_t stream, const DiagSide* side = nullptr);
hipError_t launch_decode_diag(const void* q, const void* k, const void* v, rda_dtype dt,
                              const float* alpha, const float* b, int32_t batch, int32_t heads,
                              float* S, float* o, hipStream_t stream);

// Where a prefill walk puts its outputs [T, H, 128]: fp32 rows (o), or the
// 16-bit form the fused output norm reads (y, o null).  In y each token-head
// row's 16-channel slice is scaled by a power of two, 2^(126 - E) with E the
// biased fp32 exponent of the slice's largest magnitude (so every value lies
// in (-1, 1)), and stored as fp16; in the first 8 channels of the slice the
// lowest significand bit is replaced by bit p of E, p = the channel's place
// in its slice.  E = 0 (a slice of zeros or fp32 subnormals) stands for a
// slice of zeros.
struct OutSink {
    float* o;
    uint16_t* y;
};

// Output norm and gate over `rows` rows of 128 channels: from fp32 o, or
// (o_enc) from the 16-bit form of OutSink.
int64_t norm_gate_blocks(int64_t rows);
hipError_t launch_norm_gate(const float* o, const void* g, rda_dtype g_dtype, const float* w,
                            float eps, int32_t act, int64_t rows, void* out, rda_dtype out_dtype,
                            hipStream_t stream, const uint16_t* o_enc = nullptr);

// The prep for either input type.  single_T >= 0: one sequence of single_T
// tokens without offsets, whose table the prep writes (rec_out,
// seq_off_out, num_out) instead of reading rec / num_chunks.
hipError_t launch_prep(const void* q, const void* k, rda_dtype dt,
                       const float* a, const float* b, int32_t heads, int32_t max_chunks,
                       const int32_t* rec, const int32_t* num_chunks, unsigned char* factors,
                       hipStream_t stream, int32_t single_T = -1, int32_t* rec_out = nullptr,
                       int32_t* seq_off_out = nullptr, int32_t* num_out = nullptr);

hipError_t launch_walk(const void* q, const void* k, const void* v, rda_dtype dt,
                       int32_t num_seqs, int32_t heads, const int32_t* rec,
                       const int32_t* seq_off, const int32_t* num_chunks,
                       const unsigned char* factors, const float* S0, OutSink out,
                       float* S_final, hipStream_t stream);

// Chunk `chunk`'s record for one sequence of single_T tokens and no offsets
// (plain arithmetic), written by the prep of head 0 of each chunk; chunk 0's
// also writes the sequence offsets and the chunk count nch.
__device__ __forceinline__ void prep_table_entry(int chunk, int t0, int len, int nch, int tid,
                                                 int32_t* rec_out, int32_t* seq_off_out,
                                                 int32_t* num_out) {
    if (tid < 4) {
        const int32_t field[4] = {0, t0, len, chunk};
        rec_out[4 * chunk + tid] = field[tid];
        if (chunk == 0) {
            if (tid == 0) seq_off_out[0] = 0;
            if (tid == 1) seq_off_out[1] = nch;
            if (tid == 2) num_out[0] = nch;
        }
    }
}

// bf16 prep (factors from LDS-DMA'd tiles, four workgroups per CU).  With
// single_T >= 0 the input is one sequence of single_T tokens without offsets:
// rec / num_chunks are not read, the grid covers ceil(single_T / 64) chunks,
// and the kernel writes the chunk table to rec_out / seq_off_out / num_out.
// With single_T < 0 the table in rec / num_chunks is read and the *_out
// pointers are unused.
// chunk_begin / chunk_count (single_T >= 0 only): prep just those chunks of
// the sequence (count < 0: to its end); the table entries they write carry
// the sequence's full chunk count.
hipError_t launch_prep_bf16(const uint16_t* q, const uint16_t* k, const float* a, const float* b,
                            int32_t heads, int32_t max_chunks, const int32_t* rec,
                            const int32_t* num_chunks, unsigned char* factors, int32_t single_T,
                            int32_t* rec_out, int32_t* seq_off_out, int32_t* num_out,
                            hipStream_t stream, int32_t chunk_begin = 0,
                            int32_t chunk_count = -1);

// bf16 walk (operands streamed into LDS by loader waves)

// The inputs of one bf16 prep item (rda_prep.h) and the factors' base.
struct PrepItemArgs {
    const uint16_t* q;
    const uint16_t* k;
    const float* a;
    const float* b;
    int H;
    unsigned char* factors;
};
// The output norm and gate that norm workgroups of a walk launch may run
// (after the walk's and the prep's workgroups) over rows [row_lo, row_hi)
// of the 16-bit form y (OutSink) whose walk is already done.
struct WalkNorm {
    const uint16_t* y;
    const void* g;
    int g16;                // g is bf16 (else fp32)
    const float* w;
    float eps;
    int act;                // an rda_gate_act
    void* out;
    int o16;                // out is bf16 (else fp32)
    int64_t row_lo, row_hi;
    int blocks;             // norm workgroups (0: none)
};
// Extra work a walk launch may carry: a chunk range for one sequence
// (c_hi > 0: walk chunks [c_lo, c_hi) only); prep workgroups after the
// walk's that run the prep items [item_lo, item_hi) of one sequence of
// single_T tokens and write their table entries (nch = the sequence's chunk
// count); and norm workgroups after those (WalkNorm).
struct WalkSide {
    int c_lo, c_hi;
    int prep_blocks;        // prep workgroups (0: none)
    int item_lo, item_hi;
    int single_T, nch;
    PrepItemArgs args;
    int32_t *rec_out, *seq_off_out, *num_out;
    WalkNorm norm;
    int walk_blocks;        // set by the launcher
};

// bf16 walk.  num_jobs (1 or 2) walks over the same chunks in one launch,
// differing only in their WalkJob.  seg_chunks > 0: sequence n is the n-th
// run of seg_chunks chunks of the table (segments of one sequence) instead of
// seq_off[n] .. seq_off[n + 1].  outputs = false: no output is written, and
// Q and A are not streamed.
hipError_t launch_walk_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int32_t num_seqs, int32_t heads, const int32_t* rec,
                            const int32_t* seq_off, const int32_t* num_chunks,
                            const unsigned char* factors, OutSink out, const WalkJob* jobs,
                            int32_t num_jobs, int32_t seg_chunks, bool outputs,
                            hipStream_t stream, const WalkSide* extra = nullptr);

// The segment combine of the segmented state pass, per head and value row:
// S_in[0] = S0 (zero when null); for p < P: with E_p = segment p's final
// state from zero and M_p = its transition (the final state from the
// identity with zero values),
//   S_in[p + 1] = S_in[p] M_p + E_p,
// written to S_in[p + 1] for p + 1 < P and to S_final (when not null) for
// p + 1 = P.  E, M, S_in are [P, H, 128, 128] fp32.
hipError_t launch_segment_combine(const float* S0, const float* E, const float* M, float* S_in,
                                  float* S_final, int32_t P, int32_t heads, hipStream_t stream);

}  // namespace rda
