// rda_api.hip -- the C ABI declared in include/rda.h: argument validation,
// workspace sizing and the launch sequence of each entry point.  Validation
// is pure host code and runs before anything is enqueued, so every error
// path returns a status without touching the device.
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "rda_internal.h"

using namespace rda;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range x, Range y) {
    if (x.lo == x.hi || y.lo == y.hi || x.lo == 0 || y.lo == 0) return false;
    return x.lo < y.hi && y.lo < x.hi;
}

constexpr int kWalkSlices = kD / 16;  // value-channel slices per (sequence, head)

// The segmented state pass for one long sequence with few heads.  The walk
// is sequential over chunks and gives each (sequence, head) 8 workgroups, so
// a few heads leave most of the 256 CUs idle whatever the length.  Cut into
// P segments, the sequence is walked three times as long in total but P
// times shorter in sequence: (1) every segment from zero (its end state E_p)
// and from the identity with zero values (its transition M_p) in one launch
// (2 x 8 x P x H workgroups, no outputs), (2) the combine chains the
// segments, S_in[p + 1] = S_in[p] M_p + E_p, (3) every segment again from its
// true starting state, with outputs.  Worth it when P >= 4; P fills the
// chip in the first pass and keeps segments at >= 16 chunks.
constexpr int kSegCUs = 256;
constexpr int kSegMinChunks = 16;
constexpr int kSegMax = 16;

struct SegPlan {
    int P = 0;     // segments (0: no segmented pass)
    int cps = 0;   // chunks per segment (the last may be shorter)
};

SegPlan seg_plan(int32_t num_seqs, int32_t total_tokens, int32_t heads) {
    SegPlan sp;
    if (num_seqs != 1 || total_tokens <= 0 || heads <= 0) return sp;
    const int64_t nch = (int64_t(total_tokens) + kC - 1) / kC;
    int64_t P = kSegCUs / (2 * kWalkSlices * int64_t(heads));
    P = P < nch / kSegMinChunks ? P : nch / kSegMinChunks;
    P = P < kSegMax ? P : kSegMax;
    if (P < 4) return sp;
    sp.cps = int((nch + P - 1) / P);
    sp.P = int((nch + sp.cps - 1) / sp.cps);
    return sp;
}

size_t seg_state_bytes(const SegPlan& sp, int32_t heads) {
    return size_t(sp.P) * heads * kD * kD * sizeof(float);
}

// The overlapped plan for one long sequence whose walk leaves many CUs idle
// (8 workgroups per head, one per CU), in chunk ranges: (1) the prep of the
// first range on the whole chip, (2) one launch per range whose walk
// workgroups walk it, from the state the launch before saved, while prep
// workgroups on the idle CUs prep later chunks.  When one prep item takes
// about r walk steps on one CU, the walk of L chunks hides the prep of
// g L = L idle / (r H) chunks, so each range may be g times the one before
// and the launch preps the next: the first range is short (its prep runs
// alone), the ranges grow until the last takes the rest.  r is about 3 for
// the scalar decay and about 6 for the per-channel one.  Each walk launch
// costs a ramp, and a walk slows while prep runs beside it, so growing
// ranges pay only where the prep is dear: for the per-channel decay (at
// 16384 x 16, 0.68 ms against 0.73 with two ranges).  Otherwise, and with g
// below 5/4 (many heads), two ranges: the first walk launch preps
// everything after its range, c1 = nch / (1 + g) balancing it (for the
// scalar decay at 16384 x 16 growing ranges measured 0.376-0.385 ms
// against 0.372-0.378).
//
// The fused output norm runs the norm of range i - 1 beside the walk of
// range i, on the same idle CUs, and the norm of the last range after the
// walk; for it the plan ends with a range of nch / 8 chunks (at least 16),
// long enough to hide the norm of the one before on the idle CUs.
constexpr int kOverlapMinChunks = 32;
constexpr int kOverlapMinIdleCUs = 64;
constexpr int kOverlapMaxRanges = 16;
constexpr int kOverlapMinRange = 8;
constexpr int kDiagWalkStepsPerPrepItem = 6;   // walk steps per per-channel prep item

struct OverlapPlan {
    int m = 0;            // walk launches, one per range (0: no overlap)
    int prep_blocks = 0;  // prep (or norm) workgroups beside each walk launch
    int cut[kOverlapMaxRanges + 1] = {};   // range i: chunks [cut[i], cut[i + 1])
    int pend[kOverlapMaxRanges] = {};      // chunks prepped once walk launch i ends
};

// The fused norm's last range: nch / 8 chunks, at least 16.
int64_t norm_tail_chunks(int64_t nch) { return nch / 8 > 16 ? nch / 8 : 16; }

// r walk steps per prep item; `grow`: growing ranges, the first nch / 8
// chunks; `fused`: end with the fused norm's tail range.
OverlapPlan overlap_plan(int32_t num_seqs, int32_t total_tokens, int32_t heads, bool fused,
                         int64_t r = 3, bool grow = false) {
    OverlapPlan op;
    if (num_seqs != 1 || total_tokens <= 0 || heads <= 0) return op;
    const int64_t nch = (int64_t(total_tokens) + kC - 1) / kC;
    const int64_t idle = kSegCUs - int64_t(kWalkSlices) * heads;
    if (nch < kOverlapMinChunks || idle < kOverlapMinIdleCUs) return op;
    const int64_t gn = idle, gd = r * heads;   // g = gn / gd
    const int64_t limit = nch - (fused ? norm_tail_chunks(nch) : 0);
    op.prep_blocks = int(idle);
    int m = 0;
    if (!grow || 4 * gn < 5 * gd) {
        int64_t c1 = (nch * gd + (gn + gd) / 2) / (gn + gd);
        c1 = c1 < kOverlapMinRange ? kOverlapMinRange : c1;
        c1 = c1 > nch - kOverlapMinRange ? nch - kOverlapMinRange : c1;
        op.cut[++m] = int(c1);
        if (limit >= c1 + kOverlapMinRange && limit < nch) op.cut[++m] = int(limit);
        op.cut[++m] = int(nch);
        for (int i = 0; i < m; ++i) op.pend[i] = int(nch);
        op.m = m;
        return op;
    }
    int64_t len = nch / 8 > kOverlapMinRange ? nch / 8 : kOverlapMinRange;
    while (op.cut[m] < limit) {
        int64_t next = op.cut[m] + len;
        // a short remainder joins the range before
        if (next + kOverlapMinRange > limit || m + 2 >= kOverlapMaxRanges) next = limit;
        op.cut[++m] = int(next);
        len = len * gn / gd;
    }
    if (limit < nch) op.cut[++m] = int(nch);
    for (int i = 0; i < m; ++i) op.pend[i] = op.cut[i + 2 <= m ? i + 2 : m];
    op.m = m;
    return op;
}

OverlapPlan diag_overlap_plan(int32_t num_seqs, int32_t total_tokens, int32_t heads) {
    return overlap_plan(num_seqs, total_tokens, heads, false, kDiagWalkStepsPerPrepItem, true);
}

size_t overlap_state_bytes(const OverlapPlan& op, int32_t heads) {
    return op.m > 0 ? size_t(heads) * kD * kD * sizeof(float) : 0;
}

// The 16-bit output form of the fused output norm: [T, H, 128] 16-bit values.
size_t slice_form_bytes(int32_t total_tokens, int32_t heads) {
    return align256(size_t(total_tokens > 0 ? total_tokens : 0) * size_t(heads > 0 ? heads : 0) *
                    kD * sizeof(uint16_t));
}

// Checks of the output norm's own arguments that need no sizes.
rda_status check_norm_args(rda_dtype& g_dtype, float eps, int32_t act, rda_dtype out_dtype) {
    if (out_dtype != RDA_BF16 && out_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (act != RDA_GATE_SIGMOID && act != RDA_GATE_SILU && act != RDA_GATE_NONE)
        return RDA_ERR_VALUE;
    if (act == RDA_GATE_NONE) g_dtype = RDA_BF16;   // g is not read
    if (g_dtype != RDA_BF16 && g_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (!(eps >= 0.f) || eps == INFINITY) return RDA_ERR_VALUE;
    return RDA_OK;
}

rda_status check_dims(int32_t heads, int32_t dk, int32_t dv) {
    if (heads <= 0 || dk <= 0 || dv <= 0) return RDA_ERR_SHAPE;
    if (dk != kD || dv != kD) return RDA_ERR_UNSUPPORTED;
    return RDA_OK;
}

rda_status record(hipEvent_t const* ev, int idx, hipStream_t stream) {
    if (ev && ev[idx]) {
        if (hipEventRecord(ev[idx], stream) != hipSuccess) return RDA_ERR_HIP;
    }
    return RDA_OK;
}

// Everything a prefill launch sequence needs, validated.
struct Prefill {
    const void *q, *k, *v;
    rda_dtype dt;
    const float *a, *b;
    const int32_t* cu;
    int32_t N, T, H, mc;
    const float* S0;
    float *o, *S_final;
    int32_t *rec, *seq_off, *nch;
    unsigned char* factors;
    SegPlan seg;          // used when the input is one bf16 sequence without offsets
    float *E, *F, *S_in;  // segmented pass: end states from zero, transitions, starts
    OverlapPlan ovl;      // likewise, when no segmented pass runs
    float* S_mid;         // overlapped plan: the state between walk launches
    OutSink out;          // where the walk's outputs go (o, or the slice form)
    WalkNorm norm;        // fused output norm (norm.y set): its arguments
};

rda_status check_prefill(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                         const float* a, const float* b, const int32_t* cu_seqlens,
                         int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                         int32_t dv, const float* S0, float* o, float* S_final, void* workspace,
                         size_t workspace_bytes, Prefill& P, size_t extra_ws = 0,
                         bool fused = false) {
    if (qkv_dtype != RDA_BF16 && qkv_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (total_tokens < 0 || num_seqs < 1) return RDA_ERR_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    const int32_t mc = rda_max_chunks(num_seqs, total_tokens);
    if (mc < 0) return RDA_ERR_SHAPE;
    if (int64_t(mc) * num_heads > INT32_MAX || int64_t(num_seqs) * num_heads * kWalkSlices > INT32_MAX)
        return RDA_ERR_SHAPE;
    // fused: the walk writes the slice form of the fused output norm into the
    // workspace's last extra_ws bytes instead of o (then null)
    if (total_tokens > 0 && (!q || !k || !v || !a || !b || (!o && !fused)))
        return RDA_ERR_NULL;
    if (!workspace) return RDA_ERR_WORKSPACE;
    const size_t need =
        rda_prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv) + extra_ws;
    if (workspace_bytes < need) return RDA_ERR_WORKSPACE;
    for (const void* p : {q, k, v, static_cast<const void*>(a), static_cast<const void*>(b),
                          static_cast<const void*>(S0), static_cast<const void*>(o),
                          static_cast<const void*>(S_final), static_cast<const void*>(workspace)})
        if (p && !aligned16(p)) return RDA_ERR_ALIGN;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return RDA_ERR_ALIGN;

    const size_t esz = qkv_dtype == RDA_BF16 ? 2 : 4;
    const size_t th = size_t(total_tokens) * num_heads;
    const size_t sbytes = size_t(num_seqs) * num_heads * kD * kD * sizeof(float);
    const Range rq = rng(q, th * kD * esz), rk = rng(k, th * kD * esz), rv = rng(v, th * kD * esz);
    const Range ra = rng(a, th * 4), rb = rng(b, th * 4);
    const Range ro = rng(o, th * kD * 4), rs0 = rng(S0, S0 ? sbytes : 0);
    const Range rsf = rng(S_final, S_final ? sbytes : 0), rws = rng(workspace, need);
    const Range rcu = rng(cu_seqlens, cu_seqlens ? size_t(num_seqs + 1) * 4 : 0);
    for (Range in : {rq, rk, rv, ra, rb, rs0, rcu, rsf, rws})
        if (overlap(ro, in)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ra, rb, rcu, rws})
        if (overlap(rsf, in)) return RDA_ERR_ALIAS;
    if (S0 && S_final && S0 != S_final && overlap(rs0, rsf)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ra, rb, rs0, rcu})
        if (overlap(rws, in)) return RDA_ERR_ALIAS;

    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const TableLayout tl = table_layout(mc, num_seqs);
    P = Prefill{q, k, v, qkv_dtype, a, b, cu_seqlens, num_seqs, total_tokens, num_heads, mc,
                S0, o, S_final,
                reinterpret_cast<int32_t*>(ws + tl.rec_off),
                reinterpret_cast<int32_t*>(ws + tl.seq_off_off),
                reinterpret_cast<int32_t*>(ws + tl.num_off), ws + align256(tl.bytes),
                SegPlan{}, nullptr, nullptr, nullptr, OverlapPlan{}, nullptr,
                OutSink{o, nullptr}, WalkNorm{}};
    const SegPlan sp = seg_plan(num_seqs, total_tokens, num_heads);
    const OverlapPlan op = overlap_plan(num_seqs, total_tokens, num_heads, fused);
    unsigned char* tail = P.factors + size_t(mc) * num_heads * kChunkHeadBytes;
    if (cu_seqlens == nullptr && qkv_dtype == RDA_BF16) {
        if (sp.P > 0) {
            const size_t sb = seg_state_bytes(sp, num_heads);
            P.seg = sp;
            P.E = reinterpret_cast<float*>(tail);
            P.F = reinterpret_cast<float*>(tail + sb);
            P.S_in = reinterpret_cast<float*>(tail + 2 * sb);
        } else if (op.m > 0) {
            P.ovl = op;
            P.S_mid = reinterpret_cast<float*>(tail);
        }
    }
    return RDA_OK;
}

// The overlapped plan (see overlap_plan), all on `stream`.  Stage events
// (when `ev` is given): the table stage is empty (the prep writes the
// table), the prep stage is the first launch, and the walk stage spans the
// walk launches (all but the last also prep later chunks).
rda_status prefill_overlapped(const Prefill& P, hipStream_t stream, hipEvent_t const* ev) {
    const auto* q16 = static_cast<const uint16_t*>(P.q);
    const auto* k16 = static_cast<const uint16_t*>(P.k);
    const auto* v16 = static_cast<const uint16_t*>(P.v);
    const int nch = (P.T + kC - 1) / kC;
    const OverlapPlan& op = P.ovl;
    rda_status st;
    if ((st = record(ev, 2 * RDA_STAGE_TABLE, stream)) != RDA_OK ||
        (st = record(ev, 2 * RDA_STAGE_TABLE + 1, stream)) != RDA_OK ||
        (st = record(ev, 2 * RDA_STAGE_PREP, stream)) != RDA_OK)
        return st;
    if (launch_prep_bf16(q16, k16, P.a, P.b, P.H, P.mc, nullptr, nullptr, P.factors, P.T, P.rec,
                         P.seq_off, P.nch, stream, 0, op.cut[1]) != hipSuccess)
        return RDA_ERR_HIP;
    if ((st = record(ev, 2 * RDA_STAGE_PREP + 1, stream)) != RDA_OK ||
        (st = record(ev, 2 * RDA_STAGE_WALK, stream)) != RDA_OK)
        return st;
    for (int i = 0; i < op.m; ++i) {
        // range i; beside it the prep of the chunks up to pend[i] (and their
        // table entries) and, for the fused norm, the norm of range i - 1
        WalkSide X{};
        X.c_lo = op.cut[i];
        X.c_hi = op.cut[i + 1];
        const int p_lo = i == 0 ? op.cut[1] : op.pend[i - 1];
        if (op.pend[i] > p_lo) {
            X.prep_blocks = op.prep_blocks;
            X.item_lo = p_lo * P.H;
            X.item_hi = op.pend[i] * P.H;
            X.single_T = P.T;
            X.nch = nch;
            X.args = PrepItemArgs{q16, k16, P.a, P.b, P.H, P.factors};
            X.rec_out = P.rec;
            X.seq_off_out = P.seq_off;
            X.num_out = P.nch;
        }
        if (P.norm.y && i > 0) {
            X.norm = P.norm;
            X.norm.row_lo = int64_t(kC) * op.cut[i - 1] * P.H;
            X.norm.row_hi = int64_t(kC) * op.cut[i] * P.H;
            X.norm.blocks = op.prep_blocks;
        }
        // each walk workgroup reads its slice of the saved state before it
        // writes it back, so the state between launches stays in place
        const WalkJob job{i == 0 ? P.S0 : P.S_mid, i + 1 == op.m ? P.S_final : P.S_mid, 0, 0};
        if (launch_walk_bf16(q16, k16, v16, 1, P.H, P.rec, P.seq_off, P.nch, P.factors, P.out,
                             &job, 1, 0, true, stream, &X) != hipSuccess)
            return RDA_ERR_HIP;
    }
    return record(ev, 2 * RDA_STAGE_WALK + 1, stream);
}

// Table, prep and walk one after another on `stream`, each stage bracketed
// by its event pair when `ev` is given; one bf16 sequence whose walk leaves
// CUs idle takes the overlapped plan instead.
rda_status prefill_sequential(const Prefill& P, hipStream_t stream, hipEvent_t const* ev) {
    if (P.ovl.m > 0) return prefill_overlapped(P, stream, ev);
    rda_status st;
    // one sequence without offsets: the prep kernel derives each chunk's
    // record itself and writes the table, which saves the table launch
    const bool table_in_prep = P.cu == nullptr && P.T > 0;
    if ((st = record(ev, 2 * RDA_STAGE_TABLE, stream)) != RDA_OK) return st;
    if (!table_in_prep &&
        launch_chunk_table(P.cu, P.N, P.T, P.mc, P.rec, P.seq_off, P.nch, stream) != hipSuccess)
        return RDA_ERR_HIP;
    if ((st = record(ev, 2 * RDA_STAGE_TABLE + 1, stream)) != RDA_OK) return st;
    if ((st = record(ev, 2 * RDA_STAGE_PREP, stream)) != RDA_OK) return st;
    if (table_in_prep) {
        if (launch_prep(P.q, P.k, P.dt, P.a, P.b, P.H, P.mc, nullptr, nullptr, P.factors, stream,
                        P.T, P.rec, P.seq_off, P.nch) != hipSuccess)
            return RDA_ERR_HIP;
    } else if (P.mc > 0 && P.T > 0) {
        if (launch_prep(P.q, P.k, P.dt, P.a, P.b, P.H, P.mc, P.rec, P.nch, P.factors, stream) !=
            hipSuccess)
            return RDA_ERR_HIP;
    }
    if ((st = record(ev, 2 * RDA_STAGE_PREP + 1, stream)) != RDA_OK) return st;
    if ((st = record(ev, 2 * RDA_STAGE_WALK, stream)) != RDA_OK) return st;
    if (P.seg.P > 0) {
        // the segmented pass: both first-pass jobs, the combine, the output pass
        const auto* q16 = static_cast<const uint16_t*>(P.q);
        const auto* k16 = static_cast<const uint16_t*>(P.k);
        const auto* v16 = static_cast<const uint16_t*>(P.v);
        const WalkJob first[2] = {{nullptr, P.E, 0, 0}, {nullptr, P.F, 1, 1}};
        const WalkJob last{P.S_in, nullptr, 0, 0};
        if (launch_walk_bf16(q16, k16, v16, P.seg.P, P.H, P.rec, P.seq_off, P.nch, P.factors,
                             OutSink{}, first, 2, P.seg.cps, false, stream) != hipSuccess ||
            launch_segment_combine(P.S0, P.E, P.F, P.S_in, P.S_final, P.seg.P, P.H, stream) !=
                hipSuccess ||
            launch_walk_bf16(q16, k16, v16, P.seg.P, P.H, P.rec, P.seq_off, P.nch, P.factors,
                             P.out, &last, 1, P.seg.cps, true, stream) != hipSuccess)
            return RDA_ERR_HIP;
    } else if (launch_walk(P.q, P.k, P.v, P.dt, P.N, P.H, P.rec, P.seq_off, P.nch, P.factors,
                           P.S0, P.out, P.S_final, stream) != hipSuccess) {
        return RDA_ERR_HIP;
    }
    if ((st = record(ev, 2 * RDA_STAGE_WALK + 1, stream)) != RDA_OK) return st;
    return RDA_OK;
}

// ---- the fixed scratch of rda_prefill_noalloc ------------------------------
// One array per GPU in the library's code object.  In host code `scratch`
// names a host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device may reach a kernel.
constexpr size_t kScratchBytes = RDA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// The current device's copy of `scratch`, looked up once per device.
rda_status device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RDA_ERR_HIP;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return RDA_ERR_HIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RDA_OK;
}

}  // namespace

extern "C" {

int rda_abi_version(void) { return RDA_ABI_VERSION; }

const char* rda_status_string(int status) {
    switch (status) {
        case RDA_OK: return "ok";
        case RDA_ERR_NULL: return "a required pointer is NULL";
        case RDA_ERR_SHAPE: return "invalid size argument";
        case RDA_ERR_UNSUPPORTED: return "unsupported shape (only dk = dv = 128 is implemented)";
        case RDA_ERR_DTYPE: return "unknown dtype";
        case RDA_ERR_WORKSPACE: return "workspace missing or too small";
        case RDA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case RDA_ERR_HIP: return "HIP launch error";
        case RDA_ERR_ALIAS: return "output buffers overlap other arguments";
        case RDA_ERR_VALUE: return "scalar argument out of range";
        case RDA_ERR_TOO_LARGE: return "sizes exceed the fixed scratch of rda_prefill_noalloc";
        default: return "unknown status";
    }
}

int32_t rda_max_chunks(int32_t num_seqs, int32_t total_tokens) {
    if (num_seqs < 1 || total_tokens < 0) return -1;
    const int64_t m = (int64_t(total_tokens) + int64_t(kC - 1) * num_seqs) / kC;
    if (m > INT32_MAX) return -1;
    return int32_t(m);
}

size_t rda_prefill_workspace_bytes(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                   int32_t dk, int32_t dv) {
    if (check_dims(num_heads, dk, dv) != RDA_OK) return 0;
    const int32_t mc = rda_max_chunks(num_seqs, total_tokens);
    if (mc < 0) return 0;
    const TableLayout tl = table_layout(mc, num_seqs);
    // one sequence: room for the segmented pass's three state arrays or the
    // overlapped plan's middle state
    const size_t seg = 3 * seg_state_bytes(seg_plan(num_seqs, total_tokens, num_heads), num_heads);
    const size_t mid =
        overlap_state_bytes(overlap_plan(num_seqs, total_tokens, num_heads, false), num_heads);
    return align256(tl.bytes) + size_t(mc) * size_t(num_heads) * kChunkHeadBytes +
           (seg > mid ? seg : mid);
}

rda_status rda_prefill_profiled(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                                const float* a, const float* b, const int32_t* cu_seqlens,
                                int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                int32_t dk, int32_t dv, const float* S0, float* o, float* S_final,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t const* stage_events) {
    Prefill P;
    const rda_status st = check_prefill(q, k, v, qkv_dtype, a, b, cu_seqlens, num_seqs,
                                        total_tokens, num_heads, dk, dv, S0, o, S_final,
                                        workspace, workspace_bytes, P);
    if (st != RDA_OK) return st;
    return prefill_sequential(P, stream, stage_events);
}

rda_status rda_prefill(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                       const float* a, const float* b, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                       const float* S0, float* o, float* S_final, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    Prefill P;
    const rda_status st = check_prefill(q, k, v, qkv_dtype, a, b, cu_seqlens, num_seqs,
                                        total_tokens, num_heads, dk, dv, S0, o, S_final,
                                        workspace, workspace_bytes, P);
    if (st != RDA_OK) return st;
    return prefill_sequential(P, stream, nullptr);
}

rda_status rda_prefill_noalloc(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                               const float* a, const float* b, const int32_t* cu_seqlens,
                               int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                               int32_t dk, int32_t dv, const float* S0, float* o,
                               float* S_final, hipStream_t stream) {
    // every check that needs no device first, the size against the scratch
    // included, so that an error launches nothing and touches no device
    if (qkv_dtype != RDA_BF16 && qkv_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (total_tokens < 0 || num_seqs < 1) return RDA_ERR_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    if (rda_max_chunks(num_seqs, total_tokens) < 0) return RDA_ERR_SHAPE;
    const size_t need = rda_prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv);
    if (need == 0) return RDA_ERR_SHAPE;
    if (need > kScratchBytes) return RDA_ERR_TOO_LARGE;
    void* ws = nullptr;
    if ((st = device_scratch(&ws)) != RDA_OK) return st;
    Prefill P;
    st = check_prefill(q, k, v, qkv_dtype, a, b, cu_seqlens, num_seqs, total_tokens, num_heads,
                       dk, dv, S0, o, S_final, ws, kScratchBytes, P);
    if (st != RDA_OK) return st;
    return prefill_sequential(P, stream, nullptr);
}

rda_status rda_decode_step(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                           const float* a, const float* b, int32_t batch, int32_t num_heads,
                           int32_t dk, int32_t dv, float* S, float* o, hipStream_t stream) {
    if (qkv_dtype != RDA_BF16 && qkv_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (batch < 0) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    // two workgroups per (batch, head): the grid must stay within int32
    if (int64_t(batch) * num_heads > INT32_MAX / 2) return RDA_ERR_SHAPE;
    if (batch == 0) return RDA_OK;
    if (!q || !k || !v || !a || !b || !S || !o) return RDA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(a), static_cast<const void*>(b),
                          static_cast<const void*>(S), static_cast<const void*>(o)})
        if (!aligned16(p)) return RDA_ERR_ALIGN;
    const size_t esz = qkv_dtype == RDA_BF16 ? 2 : 4;
    const size_t bh = size_t(batch) * num_heads;
    const Range rq = rng(q, bh * kD * esz), rk = rng(k, bh * kD * esz), rv = rng(v, bh * kD * esz);
    const Range ra = rng(a, bh * 4), rb = rng(b, bh * 4);
    const Range rS = rng(S, bh * kD * kD * 4), ro = rng(o, bh * kD * 4);
    for (Range in : {rq, rk, rv, ra, rb, rS})
        if (overlap(ro, in)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ra, rb})
        if (overlap(rS, in)) return RDA_ERR_ALIAS;
    if (launch_decode(q, k, v, qkv_dtype, a, b, batch, num_heads, S, o, stream) != hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

static rda_status decode_tokens_any(const void* q, const void* k, const void* v,
                                    rda_dtype qkv_dtype, const float* a, const float* b,
                                    int32_t batch, int32_t tokens, int32_t num_heads, int32_t dk,
                                    int32_t dv, const float* S_in, float* S_out,
                                    const int32_t* accept, float* o, bool diag,
                                    hipStream_t stream) {
    if (qkv_dtype != RDA_BF16 && qkv_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (batch < 0 || tokens < 0 || tokens > RDA_DECODE_MAX_TOKENS) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    if (int64_t(batch) * num_heads > INT32_MAX / 2) return RDA_ERR_SHAPE;
    if (batch == 0) return RDA_OK;
    if (!S_in || (!S_out && !o)) return RDA_ERR_NULL;
    if (tokens > 0 && (!k || !v || !a || !b || (o && !q))) return RDA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(a), static_cast<const void*>(b),
                          static_cast<const void*>(S_in), static_cast<const void*>(S_out),
                          static_cast<const void*>(o)})
        if (p && !aligned16(p)) return RDA_ERR_ALIGN;
    if (accept && (reinterpret_cast<uintptr_t>(accept) & 3u)) return RDA_ERR_ALIGN;
    const size_t esz = qkv_dtype == RDA_BF16 ? 2 : 4;
    const size_t bh = size_t(batch) * num_heads;
    const size_t th = bh * size_t(tokens);
    const Range rq = rng(o ? q : nullptr, th * kD * esz), rk = rng(k, th * kD * esz);
    const Range rv = rng(v, th * kD * esz), ra = rng(a, th * (diag ? kD : 1) * 4);
    const Range rb = rng(b, th * 4);
    const Range rsi = rng(S_in, bh * kD * kD * 4), rso = rng(S_out, bh * kD * kD * 4);
    const Range racc = rng(accept, accept ? size_t(batch) * 4 : 0), ro = rng(o, th * kD * 4);
    for (Range in : {rq, rk, rv, ra, rb, rsi, rso, racc})
        if (overlap(ro, in)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ra, rb, racc})
        if (overlap(rso, in)) return RDA_ERR_ALIAS;
    if (S_out && S_out != S_in && overlap(rso, rsi)) return RDA_ERR_ALIAS;
    // zero tokens: the only work is copying S_in to a distinct S_out
    if (tokens == 0 && (!S_out || S_out == S_in)) return RDA_OK;
    if (launch_decode_tokens(q, k, v, qkv_dtype, a, b, batch, tokens, num_heads, S_in, S_out,
                             accept, o, diag, stream) != hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

size_t rda_prefill_diag_workspace_bytes(int32_t num_seqs, int32_t total_tokens,
                                        int32_t num_heads, int32_t dk, int32_t dv) {
    if (check_dims(num_heads, dk, dv) != RDA_OK) return 0;
    const int32_t mc = rda_max_chunks(num_seqs, total_tokens);
    if (mc < 0) return 0;
    const TableLayout tl = table_layout(mc, num_seqs);
    // one sequence: room for the segmented pass's three state arrays or the
    // overlapped plan's middle state
    const size_t seg = 3 * seg_state_bytes(seg_plan(num_seqs, total_tokens, num_heads), num_heads);
    const size_t mid =
        overlap_state_bytes(diag_overlap_plan(num_seqs, total_tokens, num_heads), num_heads);
    return align256(tl.bytes) + size_t(mc) * size_t(num_heads) * kDiagChunkHeadBytes +
           (seg > mid ? seg : mid);
}

rda_status rda_prefill_diag(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                            const float* alpha, const float* b, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                            int32_t dk, int32_t dv, const float* S0, float* o, float* S_final,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (qkv_dtype != RDA_BF16 && qkv_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (total_tokens < 0 || num_seqs < 1) return RDA_ERR_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    const int32_t mc = rda_max_chunks(num_seqs, total_tokens);
    if (mc < 0) return RDA_ERR_SHAPE;
    if (int64_t(mc) * num_heads > INT32_MAX || int64_t(num_seqs) * num_heads * kWalkSlices > INT32_MAX)
        return RDA_ERR_SHAPE;
    if (total_tokens > 0 && (!q || !k || !v || !alpha || !b || !o)) return RDA_ERR_NULL;
    if (!workspace) return RDA_ERR_WORKSPACE;
    const size_t need =
        rda_prefill_diag_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv);
    if (workspace_bytes < need) return RDA_ERR_WORKSPACE;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(b),
                          static_cast<const void*>(S0), static_cast<const void*>(o),
                          static_cast<const void*>(S_final), static_cast<const void*>(workspace)})
        if (p && !aligned16(p)) return RDA_ERR_ALIGN;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return RDA_ERR_ALIGN;
    const size_t th = size_t(total_tokens) * num_heads;
    const size_t sbytes = size_t(num_seqs) * num_heads * kD * kD * sizeof(float);
    const size_t esz = qkv_dtype == RDA_BF16 ? 2 : 4;
    const Range rq = rng(q, th * kD * esz), rk = rng(k, th * kD * esz), rv = rng(v, th * kD * esz);
    const Range ral = rng(alpha, th * kD * 4), rb = rng(b, th * 4);
    const Range ro = rng(o, th * kD * 4), rs0 = rng(S0, S0 ? sbytes : 0);
    const Range rsf = rng(S_final, S_final ? sbytes : 0), rws = rng(workspace, need);
    const Range rcu = rng(cu_seqlens, cu_seqlens ? size_t(num_seqs + 1) * 4 : 0);
    for (Range in : {rq, rk, rv, ral, rb, rs0, rcu, rsf, rws})
        if (overlap(ro, in)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ral, rb, rcu, rws})
        if (overlap(rsf, in)) return RDA_ERR_ALIAS;
    if (S0 && S_final && S0 != S_final && overlap(rs0, rsf)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ral, rb, rs0, rcu})
        if (overlap(rws, in)) return RDA_ERR_ALIAS;

    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const TableLayout tl = table_layout(mc, num_seqs);
    int32_t* rec = reinterpret_cast<int32_t*>(ws + tl.rec_off);
    int32_t* seq_off = reinterpret_cast<int32_t*>(ws + tl.seq_off_off);
    int32_t* nch = reinterpret_cast<int32_t*>(ws + tl.num_off);
    if (launch_chunk_table(cu_seqlens, num_seqs, total_tokens, mc, rec, seq_off, nch, stream) !=
        hipSuccess)
        return RDA_ERR_HIP;
    unsigned char* factors = ws + align256(tl.bytes);
    const SegPlan sp = seg_plan(num_seqs, total_tokens, num_heads);
    if (sp.P > 0 && cu_seqlens == nullptr) {
        // the segmented state pass, as for rda_prefill
        unsigned char* seg = factors + size_t(mc) * num_heads * kDiagChunkHeadBytes;
        const size_t sb = seg_state_bytes(sp, num_heads);
        float* E = reinterpret_cast<float*>(seg);
        float* M = reinterpret_cast<float*>(seg + sb);
        float* S_in = reinterpret_cast<float*>(seg + 2 * sb);
        const WalkJob first[2] = {{nullptr, E, 0, 0}, {nullptr, M, 1, 1}};
        const WalkJob last{S_in, nullptr, 0, 0};
        if (launch_prep_diag(q, k, qkv_dtype, alpha, b, num_heads, mc, rec, nch, factors,
                             stream) != hipSuccess ||
            launch_walk_diag(v, qkv_dtype, sp.P, num_heads, rec, seq_off, nch, factors, nullptr,
                             first, 2, sp.cps, false, stream) != hipSuccess ||
            launch_segment_combine(S0, E, M, S_in, S_final, sp.P, num_heads, stream) !=
                hipSuccess ||
            launch_walk_diag(v, qkv_dtype, sp.P, num_heads, rec, seq_off, nch, factors, o, &last,
                             1, sp.cps, true, stream) != hipSuccess)
            return RDA_ERR_HIP;
        return RDA_OK;
    }
    const OverlapPlan op = diag_overlap_plan(num_seqs, total_tokens, num_heads);
    if (op.m > 0 && cu_seqlens == nullptr) {
        // the overlapped plan (see overlap_plan): the prep of the first range,
        // then the walk of each range beside the prep of the next on the
        // idle CUs, the state handed on in place between the walk launches
        float* S_mid = reinterpret_cast<float*>(factors + size_t(mc) * num_heads *
                                                              kDiagChunkHeadBytes);
        if (launch_prep_diag(q, k, qkv_dtype, alpha, b, num_heads, mc, rec, nch, factors, stream,
                             op.cut[1] * num_heads) != hipSuccess)
            return RDA_ERR_HIP;
        for (int i = 0; i < op.m; ++i) {
            DiagSide X{};
            X.c_lo = op.cut[i];
            X.c_hi = op.cut[i + 1];
            const int p_lo = i == 0 ? op.cut[1] : op.pend[i - 1];
            if (op.pend[i] > p_lo) {
                X.prep_blocks = op.prep_blocks;
                X.item_lo = p_lo * num_heads;
                X.item_hi = op.pend[i] * num_heads;
                X.q = q;
                X.k = k;
                X.alpha = alpha;
                X.b = b;
            }
            const WalkJob job{i == 0 ? S0 : S_mid, i + 1 == op.m ? S_final : S_mid, 0, 0};
            if (launch_walk_diag(v, qkv_dtype, 1, num_heads, rec, seq_off, nch, factors, o, &job,
                                 1, 0, true, stream, &X) != hipSuccess)
                return RDA_ERR_HIP;
        }
        return RDA_OK;
    }
    if (launch_prefill_diag(q, k, v, qkv_dtype, alpha, b, num_seqs, num_heads,
                            total_tokens > 0 ? mc : 0, rec, seq_off, nch, factors, S0, o, S_final,
                            stream) != hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

rda_status rda_decode_step_diag(const void* q, const void* k, const void* v,
                                rda_dtype qkv_dtype, const float* alpha, const float* b,
                                int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                                float* S, float* o, hipStream_t stream) {
    if (qkv_dtype != RDA_BF16 && qkv_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (batch < 0) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    if (int64_t(batch) * num_heads > INT32_MAX / 2) return RDA_ERR_SHAPE;
    if (batch == 0) return RDA_OK;
    if (!q || !k || !v || !alpha || !b || !S || !o) return RDA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(b),
                          static_cast<const void*>(S), static_cast<const void*>(o)})
        if (!aligned16(p)) return RDA_ERR_ALIGN;
    const size_t esz = qkv_dtype == RDA_BF16 ? 2 : 4;
    const size_t bh = size_t(batch) * num_heads;
    const Range rq = rng(q, bh * kD * esz), rk = rng(k, bh * kD * esz), rv = rng(v, bh * kD * esz);
    const Range ral = rng(alpha, bh * kD * 4), rb = rng(b, bh * 4);
    const Range rS = rng(S, bh * kD * kD * 4), ro = rng(o, bh * kD * 4);
    for (Range in : {rq, rk, rv, ral, rb, rS})
        if (overlap(ro, in)) return RDA_ERR_ALIAS;
    for (Range in : {rq, rk, rv, ral, rb})
        if (overlap(rS, in)) return RDA_ERR_ALIAS;
    if (launch_decode_diag(q, k, v, qkv_dtype, alpha, b, batch, num_heads, S, o, stream) !=
        hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

rda_status rda_prologue(const void* x_q, const void* x_k, const void* x_v, rda_dtype x_dtype,
                        const float* conv_w, int32_t conv_width, int32_t conv_act,
                        const void* hist_in, void* hist_out, const float* beta_raw,
                        const float* delta, const float* g_log, float decay_floor, float l2_eps,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                        int32_t num_heads, int32_t d, void* q, void* k, void* v, float* a,
                        float* b, hipStream_t stream) {
    if (x_dtype != RDA_BF16 && x_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (x_dtype != RDA_BF16) return RDA_ERR_UNSUPPORTED;
    if (conv_width < 1 || conv_width > RDA_CONV_MAX_WIDTH) return RDA_ERR_VALUE;
    if (conv_act != RDA_CONV_ACT_NONE && conv_act != RDA_CONV_ACT_SILU) return RDA_ERR_VALUE;
    if (std::isnan(decay_floor) || decay_floor == INFINITY) return RDA_ERR_VALUE;
    if (!(l2_eps >= 0.f) || l2_eps == INFINITY) return RDA_ERR_VALUE;
    if (total_tokens < 0 || num_seqs < 1) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, d, d);
    if (st != RDA_OK) return st;
    if ((num_heads + 15) / 16 > 65535) return RDA_ERR_SHAPE;   // grid y: 16 heads per block
    if (!cu_seqlens && total_tokens % num_seqs != 0) return RDA_ERR_SHAPE;
    const int32_t K = conv_width;
    const size_t hd = size_t(num_heads) * kD;
    const size_t th = size_t(total_tokens) * num_heads;
    const size_t hist_bytes = size_t(num_seqs) * 3 * (K - 1) * hd * 2;
    const bool need_hist_out = hist_out && K > 1;
    if (total_tokens == 0 && !need_hist_out) return RDA_OK;
    if (total_tokens > 0 &&
        (!x_q || !x_k || !x_v || !conv_w || !beta_raw || !g_log || !q || !k || !v || !a || !b))
        return RDA_ERR_NULL;
    for (const void* p : {x_q, x_k, x_v, static_cast<const void*>(conv_w), hist_in,
                          static_cast<const void*>(hist_out),
                          static_cast<const void*>(beta_raw), static_cast<const void*>(delta),
                          static_cast<const void*>(g_log), static_cast<const void*>(q),
                          static_cast<const void*>(k), static_cast<const void*>(v),
                          static_cast<const void*>(a), static_cast<const void*>(b)})
        if (p && !aligned16(p)) return RDA_ERR_ALIGN;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return RDA_ERR_ALIGN;
    const Range rxq = rng(x_q, th * kD * 2), rxk = rng(x_k, th * kD * 2), rxv = rng(x_v, th * kD * 2);
    const Range rw = rng(conv_w, size_t(3) * hd * K * 4);
    const Range rhi = rng(hist_in, hist_in ? hist_bytes : 0);
    const Range rho = rng(need_hist_out ? hist_out : nullptr, hist_bytes);
    const Range rbr = rng(beta_raw, th * 4), rdl = rng(delta, delta ? th * 4 : 0);
    const Range rg = rng(g_log, th * 4);
    const Range rcu = rng(cu_seqlens, cu_seqlens ? size_t(num_seqs + 1) * 4 : 0);
    const Range rq = rng(q, th * kD * 2), rk = rng(k, th * kD * 2), rv = rng(v, th * kD * 2);
    const Range ra = rng(a, th * 4), rb = rng(b, th * 4);
    const Range ins[] = {rxq, rxk, rxv, rw, rhi, rbr, rdl, rg, rcu};
    const Range outs[] = {rq, rk, rv, ra, rb, rho};
    for (int i = 0; i < 6; ++i) {
        for (Range in : ins) {
            // the history may be updated in place when every sequence has one token
            const bool hist_pair = i == 5 && in.lo == rhi.lo && in.hi == rhi.hi && rhi.lo != 0;
            if (hist_pair && !cu_seqlens && total_tokens == num_seqs) continue;
            if (overlap(outs[i], in)) return RDA_ERR_ALIAS;
        }
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return RDA_ERR_ALIAS;
    }
    PrologueArgs P;
    P.x[0] = static_cast<const uint16_t*>(x_q);
    P.x[1] = static_cast<const uint16_t*>(x_k);
    P.x[2] = static_cast<const uint16_t*>(x_v);
    P.w = conv_w;
    P.hin = static_cast<const uint16_t*>(hist_in);
    P.hout = need_hist_out ? static_cast<uint16_t*>(hist_out) : nullptr;
    P.beta = beta_raw;
    P.delta = delta;
    P.glog = g_log;
    P.floor_log = decay_floor;
    P.l2eps = l2_eps;
    P.cu = cu_seqlens;
    P.N = num_seqs;
    P.T = total_tokens;
    P.H = num_heads;
    P.L = cu_seqlens ? 0 : total_tokens / num_seqs;
    P.out[0] = static_cast<uint16_t*>(q);
    P.out[1] = static_cast<uint16_t*>(k);
    P.out[2] = static_cast<uint16_t*>(v);
    P.a = a;
    P.b = b;
    if (launch_prologue(P, K, conv_act, stream) != hipSuccess) return RDA_ERR_HIP;
    return RDA_OK;
}

rda_status rda_decode_step_prologue(const void* x_q, const void* x_k, const void* x_v,
                                   rda_dtype x_dtype, const float* conv_w, int32_t conv_width,
                                   int32_t conv_act, const void* hist_in, void* hist_out,
                                   const float* beta_raw, const float* delta, const float* g_log,
                                   float decay_floor, float l2_eps, int32_t batch,
                                   int32_t num_heads, int32_t dk, int32_t dv, float* S, float* o,
                                   hipStream_t stream) {
    if (x_dtype != RDA_BF16 && x_dtype != RDA_FP32) return RDA_ERR_DTYPE;
    if (x_dtype != RDA_BF16) return RDA_ERR_UNSUPPORTED;
    if (conv_width < 1 || conv_width > RDA_CONV_MAX_WIDTH) return RDA_ERR_VALUE;
    if (conv_act != RDA_CONV_ACT_NONE && conv_act != RDA_CONV_ACT_SILU) return RDA_ERR_VALUE;
    if (std::isnan(decay_floor) || decay_floor == INFINITY) return RDA_ERR_VALUE;
    if (!(l2_eps >= 0.f) || l2_eps == INFINITY) return RDA_ERR_VALUE;
    if (batch < 0) return RDA_ERR_SHAPE;
    rda_status st = check_dims(num_heads, dk, dv);
    if (st != RDA_OK) return st;
    if (int64_t(batch) * num_heads > INT32_MAX) return RDA_ERR_SHAPE;
    if (batch == 0) return RDA_OK;
    if (!x_q || !x_k || !x_v || !conv_w || !beta_raw || !g_log || !S || !o) return RDA_ERR_NULL;
    for (const void* p : {x_q, x_k, x_v, static_cast<const void*>(conv_w), hist_in,
                          static_cast<const void*>(hist_out), static_cast<const void*>(beta_raw),
                          static_cast<const void*>(delta), static_cast<const void*>(g_log),
                          static_cast<const void*>(S), static_cast<const void*>(o)})
        if (p && !aligned16(p)) return RDA_ERR_ALIGN;
    const int32_t K = conv_width;
    const size_t bh = size_t(batch) * num_heads;
    const size_t hist_bytes = size_t(batch) * 3 * (K - 1) * num_heads * kD * 2;
    const bool keep_hist = hist_out && K > 1;
    const Range rxq = rng(x_q, bh * kD * 2), rxk = rng(x_k, bh * kD * 2), rxv = rng(x_v, bh * kD * 2);
    const Range rw = rng(conv_w, size_t(3) * num_heads * kD * K * 4);
    const Range rhi = rng(hist_in, hist_in ? hist_bytes : 0);
    const Range rho = rng(keep_hist ? hist_out : nullptr, hist_bytes);
    const Range rbr = rng(beta_raw, bh * 4), rdl = rng(delta, delta ? bh * 4 : 0);
    const Range rg = rng(g_log, bh * 4);
    const Range rS = rng(S, bh * kD * kD * 4), ro = rng(o, bh * kD * 4);
    // the history may be updated in place (hist_out == hist_in exactly)
    const bool hist_same = keep_hist && hist_in == hist_out;
    for (Range out : {rS, ro, rho}) {
        for (Range in : {rxq, rxk, rxv, rw, rbr, rdl, rg})
            if (overlap(out, in)) return RDA_ERR_ALIAS;
    }
    if (!hist_same && overlap(rho, rhi)) return RDA_ERR_ALIAS;
    if (overlap(rS, rhi) || overlap(ro, rhi) || overlap(rS, ro) || overlap(rS, rho) ||
        overlap(ro, rho))
        return RDA_ERR_ALIAS;
    DecodePrologueArgs P;
    P.x[0] = static_cast<const uint16_t*>(x_q);
    P.x[1] = static_cast<const uint16_t*>(x_k);
    P.x[2] = static_cast<const uint16_t*>(x_v);
    P.w = conv_w;
    P.hin = static_cast<const uint16_t*>(hist_in);
    P.hout = keep_hist ? static_cast<uint16_t*>(hist_out) : nullptr;
    P.beta = beta_raw;
    P.delta = delta;
    P.glog = g_log;
    P.floor_log = decay_floor;
    P.l2eps = l2_eps;
    P.H = num_heads;
    P.S = S;
    P.o = o;
    if (launch_decode_prologue(P, batch, K, conv_act, stream) != hipSuccess) return RDA_ERR_HIP;
    return RDA_OK;
}

size_t rda_prefill_norm_gate_workspace_bytes(int32_t num_seqs, int32_t total_tokens,
                                             int32_t num_heads, int32_t dk, int32_t dv) {
    const size_t base = rda_prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv);
    if (base == 0) return 0;
    return align256(base) + slice_form_bytes(total_tokens, num_heads);
}

rda_status rda_prefill_norm_gate(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                                 const float* a, const float* b, const int32_t* cu_seqlens,
                                 int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                 int32_t dk, int32_t dv, const float* S0, const void* g,
                                 rda_dtype g_dtype, const float* weight, float eps, int32_t act,
                                 void* out, rda_dtype out_dtype, float* S_final, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    rda_status st = check_norm_args(g_dtype, eps, act, out_dtype);
    if (st != RDA_OK) return st;
    const size_t base = rda_prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv);
    const size_t extra = align256(base) - base + slice_form_bytes(total_tokens, num_heads);
    Prefill P;
    st = check_prefill(q, k, v, qkv_dtype, a, b, cu_seqlens, num_seqs, total_tokens, num_heads,
                       dk, dv, S0, nullptr, S_final, workspace, workspace_bytes, P, extra,
                       true);
    if (st != RDA_OK) return st;
    const int64_t rows = int64_t(total_tokens) * num_heads;
    if (norm_gate_blocks(rows) > INT32_MAX) return RDA_ERR_SHAPE;
    if (act == RDA_GATE_NONE) g = nullptr;
    if (rows > 0) {
        if (!out || (act != RDA_GATE_NONE && !g)) return RDA_ERR_NULL;
        for (const void* p : {g, static_cast<const void*>(weight), static_cast<const void*>(out)})
            if (p && !aligned16(p)) return RDA_ERR_ALIGN;
        const size_t n = size_t(rows) * kD;
        const size_t esz = qkv_dtype == RDA_BF16 ? 2 : 4;
        const size_t sbytes = size_t(num_seqs) * num_heads * kD * kD * sizeof(float);
        const Range rout = rng(out, n * (out_dtype == RDA_BF16 ? 2 : 4));
        const Range rg = rng(g, n * (g_dtype == RDA_BF16 ? 2 : 4));
        const Range rw = rng(weight, weight ? kD * 4 : 0);
        const Range rsf = rng(S_final, S_final ? sbytes : 0);
        const Range rws = rng(workspace, align256(base) + slice_form_bytes(total_tokens, num_heads));
        for (Range in : {rng(q, n * esz), rng(k, n * esz), rng(v, n * esz),
                         rng(a, size_t(rows) * 4), rng(b, size_t(rows) * 4),
                         rng(S0, S0 ? sbytes : 0),
                         rng(cu_seqlens, cu_seqlens ? size_t(num_seqs + 1) * 4 : 0), rg, rw, rsf,
                         rws})
            if (overlap(rout, in)) return RDA_ERR_ALIAS;
        for (Range in : {rg, rw})
            if (overlap(rsf, in) || overlap(rws, in)) return RDA_ERR_ALIAS;
    }
    unsigned char* slices = static_cast<unsigned char*>(workspace) + align256(base);
    P.out = OutSink{nullptr, reinterpret_cast<uint16_t*>(slices)};
    P.norm = WalkNorm{P.out.y, g, g_dtype == RDA_BF16 ? 1 : 0, weight, eps, act, out,
                      out_dtype == RDA_BF16 ? 1 : 0, 0, 0, 0};
    if ((st = prefill_sequential(P, stream, nullptr)) != RDA_OK) return st;
    // the overlapped plan's later walk launches have done the rows of the
    // chunks before the last walk launch's; the rest here
    const int64_t done = int64_t(kC) * (P.ovl.m > 0 ? P.ovl.cut[P.ovl.m - 1] : 0) * num_heads;
    const size_t gsz = g_dtype == RDA_BF16 ? 2 : 4, osz = out_dtype == RDA_BF16 ? 2 : 4;
    const size_t off = size_t(done) * kD;
    if (launch_norm_gate(nullptr, g ? static_cast<const unsigned char*>(g) + off * gsz : nullptr,
                         g_dtype, weight, eps, act, rows - done,
                         static_cast<unsigned char*>(out) + off * osz, out_dtype, stream,
                         P.out.y + off) != hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

rda_status rda_output_norm_gate(const float* o, const void* g, rda_dtype g_dtype,
                                const float* weight, float eps, int32_t act, int64_t rows,
                                int32_t dv, void* out, rda_dtype out_dtype, hipStream_t stream) {
    const rda_status st = check_norm_args(g_dtype, eps, act, out_dtype);
    if (st != RDA_OK) return st;
    if (rows < 0 || dv <= 0) return RDA_ERR_SHAPE;
    if (dv != kD) return RDA_ERR_UNSUPPORTED;
    if (norm_gate_blocks(rows) > INT32_MAX) return RDA_ERR_SHAPE;
    if (rows == 0) return RDA_OK;
    if (!o || !out || (act != RDA_GATE_NONE && !g)) return RDA_ERR_NULL;
    if (act == RDA_GATE_NONE) g = nullptr;
    for (const void* p : {static_cast<const void*>(o), g, static_cast<const void*>(weight),
                          static_cast<const void*>(out)})
        if (p && !aligned16(p)) return RDA_ERR_ALIGN;
    const size_t n = size_t(rows) * kD;
    const Range ro = rng(o, n * 4), rg = rng(g, n * (g_dtype == RDA_BF16 ? 2 : 4));
    const Range rw = rng(weight, weight ? kD * 4 : 0);
    const Range rout = rng(out, n * (out_dtype == RDA_BF16 ? 2 : 4));
    const bool in_place = out_dtype == RDA_FP32 && out == static_cast<const void*>(o);
    if ((!in_place && overlap(rout, ro)) || overlap(rout, rg) || overlap(rout, rw))
        return RDA_ERR_ALIAS;
    if (launch_norm_gate(o, g, g_dtype, weight, eps, act, rows, out, out_dtype, stream) !=
        hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

rda_status rda_decode_tokens(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                             const float* a, const float* b, int32_t batch, int32_t tokens,
                             int32_t num_heads, int32_t dk, int32_t dv, const float* S_in,
                             float* S_out, const int32_t* accept, float* o, hipStream_t stream) {
    return decode_tokens_any(q, k, v, qkv_dtype, a, b, batch, tokens, num_heads, dk, dv, S_in,
                             S_out, accept, o, false, stream);
}

rda_status rda_decode_tokens_diag(const void* q, const void* k, const void* v,
                                  rda_dtype qkv_dtype, const float* alpha, const float* b,
                                  int32_t batch, int32_t tokens, int32_t num_heads, int32_t dk,
                                  int32_t dv, const float* S_in, float* S_out,
                                  const int32_t* accept, float* o, hipStream_t stream) {
    return decode_tokens_any(q, k, v, qkv_dtype, alpha, b, batch, tokens, num_heads, dk, dv,
                             S_in, S_out, accept, o, true, stream);
}

rda_status rda_chunk_table(const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                           int32_t* out, int32_t* out_seq_offsets, int32_t* out_num_chunks,
                           hipStream_t stream) {
    if (total_tokens < 0 || num_seqs < 1) return RDA_ERR_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return RDA_ERR_SHAPE;
    const int32_t mc = rda_max_chunks(num_seqs, total_tokens);
    if (mc < 0) return RDA_ERR_SHAPE;
    if (!out_seq_offsets || !out_num_chunks || (mc > 0 && !out)) return RDA_ERR_NULL;
    for (const void* p : {static_cast<const void*>(cu_seqlens), static_cast<const void*>(out),
                          static_cast<const void*>(out_seq_offsets),
                          static_cast<const void*>(out_num_chunks)})
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return RDA_ERR_ALIGN;
    if (launch_chunk_table(cu_seqlens, num_seqs, total_tokens, mc, out, out_seq_offsets,
                           out_num_chunks, stream) != hipSuccess)
        return RDA_ERR_HIP;
    return RDA_OK;
}

}  // extern "C"
