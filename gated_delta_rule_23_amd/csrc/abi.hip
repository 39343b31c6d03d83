// abi.hip -- the extern "C" boundary of libgdr (declared in include/gdr.h).
//
// Every entry point validates its arguments completely before touching the
// HIP runtime, so a rejected call enqueues nothing and needs no GPU. Errors
// are integer status codes plus a per-thread message (gdr_last_error).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "gdr.h"
#include "kernels.hpp"
#include "norm_la.hpp"

// The workspace of gdr_chunk_fwd_noalloc: one array per GPU, allocated when
// the library's code is loaded on that GPU and held until the process ends.
// Host code never passes its name to a kernel or a copy (on the host it only
// names the symbol); it uses the device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return GDR_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(GDR_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(GDR_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(GDR_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GDR_OK;
}

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

// Largest element count of any [B, T, H, D] array must fit comfortably in
// 64-bit offsets and in the 31-bit grid dimensions used by the launches.
bool size_ok(long long B, long long T, long long H, long long D) {
    const long long lim = (long long)1 << 40;
    return B <= lim && T <= lim && H <= lim && D <= lim && B * T <= lim && B * T * H <= lim && B * T * H * D <= lim;
}

// Checks shared by every compute call. Decode has no T axis; the chunked
// prefill also checks the chunk length and its supported dtypes.
enum CallKind { CALL_DECODE, CALL_CHUNK, CALL_RECURRENT, CALL_CHUNK_BWD };
int validate(const gdr_desc *d, CallKind kind, const void *q, const void *k, const void *v, const float *g,
             const float *beta, const void *b, const void *w, const void *o) {
    const bool prefill = kind != CALL_DECODE;
    if (!d) return fail(GDR_E_INVAL, "desc is NULL");
    if (d->B < 0) return fail(GDR_E_INVAL, "B = %d must be >= 0", d->B);
    if (prefill && d->T < 0) return fail(GDR_E_INVAL, "T = %d must be >= 0", d->T);
    if (d->H_qk <= 0 || d->H_v <= 0) return fail(GDR_E_INVAL, "H_qk = %d and H_v = %d must be > 0", d->H_qk, d->H_v);
    if (d->H_v % d->H_qk != 0)
        return fail(GDR_E_INVAL, "H_v = %d must be a multiple of H_qk = %d", d->H_v, d->H_qk);
    if (d->d_k <= 0 || d->d_v <= 0) return fail(GDR_E_INVAL, "d_k = %d and d_v = %d must be > 0", d->d_k, d->d_v);
    if (d->io_dtype != GDR_F32 && d->io_dtype != GDR_BF16) return fail(GDR_E_INVAL, "io_dtype = %d", d->io_dtype);
    if (d->decay < GDR_DECAY_NONE || d->decay > GDR_DECAY_CHANNEL) return fail(GDR_E_INVAL, "decay = %d", d->decay);
    if (!std::isfinite(d->scale)) return fail(GDR_E_INVAL, "scale must be finite");
    if (d->d_k != d->d_v || !supported_dim(d->d_k))
        return fail(GDR_E_UNSUPPORTED, "d_k = %d, d_v = %d: supported are d_k == d_v in {32, 64, 128}", d->d_k, d->d_v);
    if (kind == CALL_CHUNK || kind == CALL_CHUNK_BWD) {
        if (d->chunk != gdr::kChunk) return fail(GDR_E_UNSUPPORTED, "chunk = %d: only 64 is supported", d->chunk);
        if (kind == CALL_CHUNK && !gdr::chunk_supported(d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32, d->d_k))
            return fail(GDR_E_UNSUPPORTED, "prefill with float32 io supports d in {32, 64, 128}");
    }
    if (!size_ok(d->B, prefill ? d->T : 1, d->H_v, d->d_k) || !size_ok(d->B, prefill ? d->T : 1, d->H_qk, d->d_k))
        return fail(GDR_E_INVAL, "sizes too large");
    // An empty call (no sequences, or no tokens) reads and writes no per-token
    // array, so those pointers may be NULL (empty tensors have no storage).
    if (d->B == 0 || (prefill && d->T == 0)) return GDR_OK;
    if (!q || !k || !v || !o) return fail(GDR_E_INVAL, "q, k, v and o must be non-NULL");
    if ((d->decay == GDR_DECAY_NONE) != (g == nullptr))
        return fail(GDR_E_INVAL, "g must be NULL exactly when decay is GDR_DECAY_NONE");
    if (beta) {
        if (b || w) return fail(GDR_E_INVAL, "beta given: b and w must be NULL (tied gates)");
    } else {
        if (!b || !w) return fail(GDR_E_INVAL, "beta NULL: both b and w must be given (decoupled gates)");
    }
    return GDR_OK;
}

// The kernels read and write the io arrays, the state and the workspace with
// 16-byte vector accesses; beta and a scalar decay are read per element.
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool overlap(const void *x, const void *y, size_t n) {
    const char *a = static_cast<const char *>(x), *b = static_cast<const char *>(y);
    return a < b + n && b < a + n;
}
int check_alignment(const gdr_desc *d, std::initializer_list<const void *> vec16, const float *g, const float *beta) {
    for (const void *p : vec16)
        if (p && !aligned(p, 16)) return fail(GDR_E_INVAL, "array pointers must be 16-byte aligned");
    if (g && !aligned(g, d->decay == GDR_DECAY_CHANNEL ? 16 : 4)) return fail(GDR_E_INVAL, "g is misaligned");
    if (beta && !aligned(beta, 4)) return fail(GDR_E_INVAL, "beta is misaligned");
    return GDR_OK;
}

// Bytes of one convolution state [B, 3, (2 H_qk + H_v) d] in the io dtype.
size_t conv_state_bytes(const gdr_desc *d) {
    return (size_t)d->B * 3 * (2 * (size_t)d->H_qk + d->H_v) * d->d_k * (d->io_dtype == GDR_BF16 ? 2 : 4);
}

// The input stage's own checks (stage may be NULL: no input stage).
int check_stage(const gdr_desc *d, const gdr_input_stage *stage) {
    if (!stage) return GDR_OK;
    if (!stage->conv_w) return fail(GDR_E_INVAL, "the input stage needs conv_w");
    if (!aligned(stage->conv_w, 16) || (stage->conv_in && !aligned(stage->conv_in, 16)) ||
        (stage->conv_out && !aligned(stage->conv_out, 16)) || (stage->decay_scale && !aligned(stage->decay_scale, 4)))
        return fail(GDR_E_INVAL, "input-stage arrays are misaligned");
    if (stage->conv_in && stage->conv_out && overlap(stage->conv_in, stage->conv_out, conv_state_bytes(d)))
        return fail(GDR_E_INVAL, "conv_out must not overlap conv_in");
    return GDR_OK;
}

// Byte ranges [x, x + nx) and [y, y + ny) intersect.
bool ranges_meet(const void *x, size_t nx, const void *y, size_t ny) {
    const char *a = static_cast<const char *>(x), *b = static_cast<const char *>(y);
    return nx && ny && a < b + ny && b < a + nx;
}

// The chunked prefill's aliasing rules: S_T equals S0 or does not overlap
// it (one sweep workgroup's state writes would otherwise land on entries
// another has yet to read), and o, S_T (unless it is S0) and the workspace
// overlap no input and no other output.
int check_chunk_overlaps(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const void *b, const void *w, const float *S0, const void *o,
                         const float *ST, const void *ws, size_t ws_bytes) {
    if (d->B == 0) return GDR_OK;
    const size_t esz = d->io_dtype == GDR_BF16 ? 2 : 4, D = d->d_k, tok = (size_t)d->B * d->T;
    const size_t sbytes = (size_t)d->B * d->H_v * D * D * sizeof(float);
    struct Range { const void *p; size_t n; };
    const Range in[] = {{q, tok * d->H_qk * D * esz},
                        {k, tok * d->H_qk * D * esz},
                        {v, tok * d->H_v * D * esz},
                        {g, g ? tok * d->H_v * (d->decay == GDR_DECAY_CHANNEL ? D : 1) * sizeof(float) : 0},
                        {beta, beta ? tok * d->H_v * sizeof(float) : 0},
                        {b, b ? tok * d->H_v * D * esz : 0},
                        {w, w ? tok * d->H_v * D * esz : 0},
                        {S0, S0 ? sbytes : 0}};
    const Range out[] = {{o, tok * d->H_v * D * esz}, {ST, sbytes}, {ws, ws ? ws_bytes : 0}};
    const char *name[] = {"o", "ST", "the workspace"};
    for (int i = 0; i < 3; ++i) {
        if (!out[i].p) continue;
        for (const Range &x : in) {
            if (i == 1 && x.p == S0 && ST == S0) continue;  // S_T may be S0 itself
            if (x.p && ranges_meet(out[i].p, out[i].n, x.p, x.n)) {
                if (i == 1 && x.p == S0) return fail(GDR_E_INVAL, "ST must equal S0 or not overlap it");
                return fail(GDR_E_INVAL, "%s overlaps an input", name[i]);
            }
        }
        for (int j = i + 1; j < 3; ++j)
            if (out[j].p && ranges_meet(out[i].p, out[i].n, out[j].p, out[j].n))
                return fail(GDR_E_INVAL, "%s overlaps %s", name[i], name[j]);
    }
    return GDR_OK;
}

// lib_scratch: the workspace is the library's own `scratch` array (the
// workspace arguments are ignored).
int chunk_call(const gdr_desc *d, const gdr_input_stage *stage, const void *q, const void *k, const void *v,
                      const float *g, const float *beta, const void *b, const void *w, const float *S0, void *o,
                      float *ST, void *workspace, size_t workspace_bytes, void *stream, bool lib_scratch = false) {
    int rc = validate(d, CALL_CHUNK, q, k, v, g, beta, b, w, o);
    if (rc != GDR_OK) return rc;
    if (!ST) return fail(GDR_E_INVAL, "ST must be non-NULL");
    rc = check_alignment(d, {q, k, v, b, w, o, S0, ST, workspace}, g, beta);
    if (rc != GDR_OK) return rc;
    rc = check_stage(d, stage);
    if (rc != GDR_OK) return rc;
    const int io = d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32;
    const int NC = (d->T + gdr::kChunk - 1) / gdr::kChunk;
    const bool chan = d->decay == GDR_DECAY_CHANNEL;
    if (io == gdr::IO_F32 && d->d_k == 128 && (chan || !beta || stage))
        return fail(GDR_E_UNSUPPORTED, "prefill with float32 io at d = 128 supports tied gates (beta) with a scalar "
                                       "decay or none, without the input stage");
    const gdr::ChunkWsLayout L = gdr::chunk_ws_layout(d->B, d->H_qk, d->H_v, NC, d->d_k, io, chan);
    // Per-channel decay with the input stage: the convolution and the
    // normalisation of q, k, v run as a pass of their own into the workspace,
    // after the prefill's part; the prefill applies the gate and decay
    // activations as it loads them.
    const bool split_stage = stage && chan;
    const gdr::StageWsLayout SL = gdr::stage_ws_layout(d->B, d->T, d->H_qk, d->H_v, d->d_k, io);
    const size_t need = L.total() + (split_stage ? SL.total() : 0);
    if (lib_scratch) {
        workspace = nullptr;
        if (need > GDR_NOALLOC_SCRATCH_BYTES)
            return fail(GDR_E_UNSUPPORTED, "workspace of %zu bytes needed; the library's scratch holds %zu",
                        need, (size_t)GDR_NOALLOC_SCRATCH_BYTES);
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return fail(GDR_E_INVAL, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    }
    rc = check_chunk_overlaps(d, q, k, v, g, beta, b, w, S0, o, ST, workspace, need);
    if (rc != GDR_OK) return rc;
    if (d->B == 0) return ok();
    const size_t units = (size_t)d->B * d->H_v * NC;
    if (units > 0x7fffffffull) return fail(GDR_E_UNSUPPORTED, "too many chunks for one launch");
    if (lib_scratch) {
        rc = scratch_of_current_device(&workspace);
        if (rc != GDR_OK) return rc;
    }

    gdr::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.bg = b; a.wg = w;
    a.S0 = S0; a.o = o; a.ST = ST;
    a.ws_io = workspace;
    a.ws_tab = reinterpret_cast<float *>(static_cast<char *>(workspace) + L.io_bytes);
    a.ws_kT = L.kT_bytes ? static_cast<char *>(workspace) + L.io_bytes + L.tab_bytes : nullptr;
    a.ws_seg = L.seg_bytes ? reinterpret_cast<float *>(static_cast<char *>(workspace) + L.io_bytes + L.tab_bytes +
                                                       L.kT_bytes)
                           : nullptr;
    gdr::chunk_segments(d->B, d->H_v, d->d_k, NC, io, a.P, a.L);
    a.B = d->B; a.T = d->T; a.Hqk = d->H_qk; a.Hv = d->H_v; a.decay = d->decay; a.NC = NC;
    a.scale = d->scale;
    hipError_t e = hipSuccess;
    if (split_stage && NC > 0) {
        char *p = static_cast<char *>(workspace) + L.total();
        gdr::StageArgs sa{};
        sa.q = q; sa.k = k; sa.v = v;
        sa.conv_w = stage->conv_w; sa.conv_in = stage->conv_in; sa.conv_out = stage->conv_out;
        sa.qo = p;
        sa.ko = p + SL.qk;
        sa.vo = p + 2 * SL.qk;
        sa.B = d->B; sa.T = d->T; sa.Hqk = d->H_qk; sa.Hv = d->H_v;
        e = gdr::launch_stage(io, d->d_k, sa, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "input stage launch");
        a.q = sa.qo; a.k = sa.ko; a.v = sa.vo;
        a.raw_gates = 1;
        a.decay_scale = stage->decay_scale;
    } else if (stage) {
        a.conv_w = stage->conv_w;
        a.conv_in = stage->conv_in;
        a.conv_out = stage->conv_out;
        a.decay_scale = stage->decay_scale;
    }
    e = gdr::launch_chunk(io, d->d_k, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "chunk prefill launch");
    if (stage && stage->conv_out && NC == 0) {  // no chunk: the state passes through unchanged
        e = gdr::launch_state_fill(static_cast<float *>(stage->conv_out), static_cast<const float *>(stage->conv_in),
                                   conv_state_bytes(d) / sizeof(float), static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "convolution state copy");
    }
    return ok();
}

int recurrent_call(const gdr_desc *d, const gdr_input_stage *stage, const void *q, const void *k,
                          const void *v, const float *g, const float *beta, const void *b, const void *w,
                          const float *S0, void *o, float *ST, void *stream) {
    int rc = validate(d, CALL_RECURRENT, q, k, v, g, beta, b, w, o);
    if (rc != GDR_OK) return rc;
    if (!ST) return fail(GDR_E_INVAL, "ST must be non-NULL");
    rc = check_alignment(d, {q, k, v, b, w, o, S0, ST}, g, beta);
    if (rc != GDR_OK) return rc;
    if (S0 && S0 != ST) {
        const size_t n = gdr_state_bytes(d->B, d->H_v, d->d_k, d->d_v);
        if (overlap(S0, ST, n)) return fail(GDR_E_INVAL, "ST must equal S0 or not overlap it");
    }
    rc = check_stage(d, stage);
    if (rc != GDR_OK) return rc;
    if (d->B == 0) return ok();
    // At most two workgroups per (sequence, V head).
    if ((long long)d->B * d->H_v * 2 > 0x7fffffffll) return fail(GDR_E_UNSUPPORTED, "B * H_v too large for one launch");
    gdr::RecurArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.bg = b; a.wg = w;
    a.S0 = S0; a.ST = ST; a.o = o;
    a.B = d->B; a.T = d->T; a.Hqk = d->H_qk; a.Hv = d->H_v; a.decay = d->decay; a.scale = d->scale;
    if (stage) {
        a.conv_w = stage->conv_w;
        a.conv_in = stage->conv_in;
        a.conv_out = stage->conv_out;
        a.decay_scale = stage->decay_scale;
    }
    hipError_t e = gdr::launch_recurrent(d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32, d->d_k, a,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "recurrent launch");
    return ok();
}

// Byte ranges: an output must overlap neither another output nor any input
// (NULL or empty ranges are skipped).
struct Span {
    const void *p;
    size_t n;
};
bool spans_overlap(const Span &x, const Span &y) {
    if (!x.p || !x.n || !y.p || !y.n) return false;
    const char *a = static_cast<const char *>(x.p), *b = static_cast<const char *>(y.p);
    return a < b + y.n && b < a + x.n;
}
bool any_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto x = outs.begin(); x != outs.end(); ++x) {
        for (auto y = x + 1; y != outs.end(); ++y)
            if (spans_overlap(*x, *y)) return true;
        for (const Span &y : ins)
            if (spans_overlap(*x, y)) return true;
    }
    return false;
}

size_t bwd_workspace(const gdr_desc *d, bool chunked) {
    return chunked ? gdr::chunk_bwd_ws_layout(d->B, d->T, d->H_qk, d->H_v, d->d_k).total()
                   : gdr::bwd_ws_layout(d->B, d->T, d->H_v, d->d_k).total();
}

int bwd_workspace_bytes(const gdr_desc *d, size_t *bytes, bool chunked) {
    if (!bytes) return fail(GDR_E_INVAL, "bytes is NULL");
    *bytes = 0;
    static const char dummy = 0;
    const void *p = &dummy;
    const int rc = validate(d, chunked ? CALL_CHUNK_BWD : CALL_RECURRENT, p, p, p,
                            d && d->decay != GDR_DECAY_NONE ? (const float *)p : nullptr, (const float *)p, nullptr,
                            nullptr, p);
    if (rc != GDR_OK) return rc;
    *bytes = bwd_workspace(d, chunked);
    return ok();
}

int bwd_call(bool chunked, const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
             const float *beta, const void *b, const void *w, const float *S0, const void *dO, const float *dST,
             float *dq, float *dk, float *dv, float *dg, float *dbeta, float *db, float *dw, float *dS0,
             void *workspace, size_t workspace_bytes, void *stream) {
    if (d && d->B > 0 && d->T > 0 && !dO) return fail(GDR_E_INVAL, "dO must be non-NULL");
    int rc = validate(d, chunked ? CALL_CHUNK_BWD : CALL_RECURRENT, q, k, v, g, beta, b, w, dO);
    if (rc != GDR_OK) return rc;
    rc = check_alignment(d, {q, k, v, b, w, dO, S0, dST, dq, dk, dv, db, dw, dS0, workspace}, g, beta);
    if (rc != GDR_OK) return rc;
    const bool chan = d->decay == GDR_DECAY_CHANNEL;
    if ((dg && !aligned(dg, chan ? 16 : 4)) || (dbeta && !aligned(dbeta, 4)))
        return fail(GDR_E_INVAL, "dg or dbeta is misaligned");
    const size_t BT = (size_t)d->B * d->T, D = d->d_k;
    const size_t esz = d->io_dtype == GDR_BF16 ? 2 : 4;
    const size_t nqk = BT * d->H_qk * D, nv = BT * d->H_v * D, nh = BT * d->H_v;
    const size_t state = gdr_state_bytes(d->B, d->H_v, d->d_k, d->d_v);
    const size_t wsb = bwd_workspace(d, chunked);
    if (d->B > 0 && d->T > 0) {
        if (!dq || !dk || !dv) return fail(GDR_E_INVAL, "dq, dk and dv must be non-NULL");
        if ((g == nullptr) != (dg == nullptr)) return fail(GDR_E_INVAL, "dg must be given exactly when g is");
        if ((beta == nullptr) != (dbeta == nullptr)) return fail(GDR_E_INVAL, "dbeta must be given exactly when beta is");
        if ((b == nullptr) != (db == nullptr) || (w == nullptr) != (dw == nullptr))
            return fail(GDR_E_INVAL, "db and dw must be given exactly when b and w are");
        if (!workspace || workspace_bytes < wsb)
            return fail(GDR_E_INVAL, "workspace of %zu bytes needed, %zu given", wsb, workspace ? workspace_bytes : 0);
    }
    const size_t ng = g ? (chan ? nv : nh) * 4 : 0;
    if (any_overlap({{dq, nqk * 4}, {dk, nqk * 4}, {dv, nv * 4}, {dg, ng}, {dbeta, dbeta ? nh * 4 : 0},
                     {db, db ? nv * 4 : 0}, {dw, dw ? nv * 4 : 0}, {dS0, dS0 ? state : 0}},
                    {{q, nqk * esz}, {k, nqk * esz}, {v, nv * esz}, {g, ng}, {beta, beta ? nh * 4 : 0},
                     {b, b ? nv * esz : 0}, {w, w ? nv * esz : 0}, {S0, S0 ? state : 0}, {dO, nv * esz},
                     {dST, dST ? state : 0}, {workspace, workspace ? wsb : 0}}))
        return fail(GDR_E_INVAL, "gradient arrays must not overlap one another, the inputs or the workspace");
    if (d->B == 0) return ok();
    const long long chunks = ((long long)d->T + gdr::kChunk - 1) / gdr::kChunk;
    if ((long long)d->B * d->H_v * (d->d_k / gdr::kBwdCols) > 0x7fffffffll ||
        (long long)d->B * d->T * d->H_qk > 0x7fffffffll || (chunked && (long long)d->B * d->H_v * chunks > 0x7fffffffll))
        return fail(GDR_E_UNSUPPORTED, "too many work items for one launch");
    if (d->T == 0) {  // no token: the gradient reaching S0 is dL/dS_T itself
        if (dS0) {
            hipError_t e = gdr::launch_state_fill(dS0, dST, state / sizeof(float), static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e, "dS0 copy");
        }
        return ok();
    }
    const int io = d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32;
    hipError_t e;
    if (chunked) {
        gdr::ChunkBwdArgs a{};
        a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.bg = b; a.wg = w; a.S0 = S0; a.dO = dO; a.dST = dST;
        a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.db = db; a.dw = dw; a.dS0 = dS0;
        const gdr::ChunkBwdWsLayout L = gdr::chunk_bwd_ws_layout(d->B, d->T, d->H_qk, d->H_v, d->d_k);
        float **arr[gdr::kChunkBwdArrays] = {&a.wUz, &a.wQt, &a.wU, &a.wdU, &a.wdE, &a.wdQ, &a.wdK,
                                             &a.wA, &a.wT, &a.wdA, &a.wdT, &a.wS, &a.wdS, &a.wG, &a.wGam, &a.wdGam,
                                             &a.wdq, &a.wdk, &a.wYt, &a.wKet};
        char *p = static_cast<char *>(workspace);
        for (int i = 0; i < gdr::kChunkBwdArrays; ++i) {
            *arr[i] = L.floats[i] ? reinterpret_cast<float *>(p) : nullptr;
            p += gdr::align256(L.floats[i] * 4);
        }
        a.wP = a.wdE;  // p and b of the backward sweep (see ChunkBwdArgs); wdK follows wdQ directly
        a.wB = a.wdQ;
        a.B = d->B; a.T = d->T; a.Hqk = d->H_qk; a.Hv = d->H_v; a.decay = d->decay; a.scale = d->scale;
        a.NC = (int)chunks;
        e = gdr::launch_chunk_backward(io, d->d_k, a, static_cast<hipStream_t>(stream));
    } else {
        const gdr::BwdWsLayout L = gdr::bwd_ws_layout(d->B, d->T, d->H_v, d->d_k);
        gdr::BwdArgs a{};
        a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.bg = b; a.wg = w; a.S0 = S0; a.dO = dO; a.dST = dST;
        a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.db = db; a.dw = dw; a.dS0 = dS0;
        a.ws_ck = static_cast<float *>(workspace);
        a.ws_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + L.ck_bytes);
        a.B = d->B; a.T = d->T; a.Hqk = d->H_qk; a.Hv = d->H_v; a.decay = d->decay; a.scale = d->scale;
        e = gdr::launch_backward(io, d->d_k, a, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return ok();
}

// Normalised linear attention: checks shared by the prefill and the decode
// step (T = 1 for decode). S0/z0 and ST/zT may be the same arrays.
int nla_call(const gdr_desc *d, bool decode, const void *q, const void *k, const void *v, const float *S0,
             const float *z0, void *o, float *ST, float *zT, void *ws, size_t ws_bytes, void *stream) {
    if (!d) return fail(GDR_E_INVAL, "desc is NULL");
    const int T = decode ? 1 : d->T;
    if (d->B < 0) return fail(GDR_E_INVAL, "B = %d must be >= 0", d->B);
    if (T < 0) return fail(GDR_E_INVAL, "T = %d must be >= 0", T);
    if (d->H_qk <= 0 || d->H_v <= 0) return fail(GDR_E_INVAL, "H_qk = %d and H_v = %d must be > 0", d->H_qk, d->H_v);
    if (d->H_v % d->H_qk != 0)
        return fail(GDR_E_INVAL, "H_v = %d must be a multiple of H_qk = %d", d->H_v, d->H_qk);
    if (d->io_dtype != GDR_F32 && d->io_dtype != GDR_BF16) return fail(GDR_E_INVAL, "io_dtype = %d", d->io_dtype);
    if (d->decay != GDR_DECAY_NONE) return fail(GDR_E_INVAL, "normalised linear attention has no decay: decay must be GDR_DECAY_NONE");
    if (d->d_k != d->d_v || !supported_dim(d->d_k))
        return fail(GDR_E_UNSUPPORTED, "d_k = %d, d_v = %d: supported are d_k == d_v in {32, 64, 128}", d->d_k, d->d_v);
    if (!decode && d->chunk != gdr::kChunk) return fail(GDR_E_UNSUPPORTED, "chunk = %d: only 64 is supported", d->chunk);
    if (!size_ok(d->B, T, d->H_v, d->d_k)) return fail(GDR_E_INVAL, "sizes too large");
    if (d->B == 0) return ok();
    if (!ST || !zT) return fail(GDR_E_INVAL, decode ? "S and z must be non-NULL" : "ST and zT must be non-NULL");
    if (T > 0 && (!q || !k || !v || !o)) return fail(GDR_E_INVAL, "phq, phk, v and o must be non-NULL");
    for (const void *p : std::initializer_list<const void *>{q, k, v, o, S0, z0, ST, zT, ws})
        if (p && !aligned(p, 16)) return fail(GDR_E_INVAL, "array pointers must be 16-byte aligned");
    const int D = d->d_k, NC = (T + gdr::kChunk - 1) / gdr::kChunk;
    const size_t need = gdr::nla_ws_bytes(d->B, d->H_v, D, NC);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(GDR_E_INVAL, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    // Outputs against inputs and one another (S_T may be S0, z_T may be z0).
    const size_t esz = d->io_dtype == GDR_BF16 ? 2 : 4, tok = (size_t)d->B * T;
    const size_t sb = (size_t)d->B * d->H_v * D * D * sizeof(float), zb = (size_t)d->B * d->H_v * D * sizeof(float);
    struct Range { const void *p; size_t n; };
    const Range in[] = {{q, tok * d->H_qk * D * esz}, {k, tok * d->H_qk * D * esz}, {v, tok * d->H_v * D * esz},
                        {S0, S0 ? sb : 0}, {z0, z0 ? zb : 0}};
    const Range out[] = {{o, T > 0 ? tok * d->H_v * D * esz : 0}, {ST, sb}, {zT, zb}, {ws, need}};
    const char *name[] = {"o", "ST", "zT", "the workspace"};
    for (int i = 0; i < 4; ++i) {
        if (!out[i].p || !out[i].n) continue;
        for (const Range &x : in) {
            if (!x.p || !x.n || (i == 1 && x.p == S0 && ST == S0) || (i == 2 && x.p == z0 && zT == z0)) continue;
            if (ranges_meet(out[i].p, out[i].n, x.p, x.n))
                return fail(GDR_E_INVAL, "%s overlaps an input (ST may equal S0 and zT z0, nothing else)", name[i]);
        }
        for (int j = i + 1; j < 4; ++j)
            if (out[j].p && out[j].n && ranges_meet(out[i].p, out[i].n, out[j].p, out[j].n))
                return fail(GDR_E_INVAL, "%s overlaps %s", name[i], name[j]);
    }
    gdr::NlaArgs a{};
    a.q = q; a.k = k; a.v = v; a.S0 = S0; a.z0 = z0; a.o = o; a.ST = ST; a.zT = zT;
    a.ws = static_cast<float *>(ws);
    a.B = d->B; a.T = T; a.Hqk = d->H_qk; a.Hv = d->H_v; a.NC = NC;
    gdr::nla_segments(d->B, d->H_v, D, NC, a.P, a.L);
    a.z_apart = !decode && a.P == 1 && z0 && z0 == zT;
    const hipError_t e = gdr::launch_nla(d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32, D, a, decode,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "normalised linear attention launch");
    return ok();
}

}  // namespace

extern "C" {

const char *gdr_last_error(void) { return g_err.c_str(); }

int gdr_version(void) { return 1; }

size_t gdr_state_bytes(int B, int H_v, int d_k, int d_v) {
    if (B <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0) return 0;
    return (size_t)B * H_v * d_k * d_v * sizeof(float);
}

int gdr_state_alloc(int B, int H_v, int d_k, int d_v, float **state, size_t *bytes, void *stream) {
    if (!state) return fail(GDR_E_INVAL, "state is NULL");
    *state = nullptr;
    const size_t n = gdr_state_bytes(B, H_v, d_k, d_v);
    if (n == 0) return fail(GDR_E_INVAL, "sizes must be > 0");
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, n);
    if (e != hipSuccess) return fail(GDR_E_NOMEM, "hipMalloc(%zu): %s", n, hipGetErrorString(e));
    e = gdr::launch_state_fill(static_cast<float *>(p), nullptr, n / sizeof(float), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        (void)hipFree(p);
        return hip_fail(e, "zero fill");
    }
    *state = static_cast<float *>(p);
    if (bytes) *bytes = n;
    return ok();
}

int gdr_state_free(float *state) {
    if (!state) return ok();
    hipError_t e = hipFree(state);
    if (e != hipSuccess) return hip_fail(e, "hipFree");
    return ok();
}

int gdr_chunk_workspace_bytes(const gdr_desc *d, size_t *bytes) {
    if (!bytes) return fail(GDR_E_INVAL, "bytes is NULL");
    *bytes = 0;
    // Pointers are not known here; validate the sizes with dummy non-NULL pointers.
    static const char dummy = 0;
    const void *p = &dummy;
    const int rc = validate(d, CALL_CHUNK, p, p, p, d && d->decay != GDR_DECAY_NONE ? (const float *)p : nullptr,
                            (const float *)p, nullptr, nullptr, p);
    if (rc != GDR_OK) return rc;
    const int NC = (d->T + gdr::kChunk - 1) / gdr::kChunk;
    *bytes = gdr::chunk_ws_layout(d->B, d->H_qk, d->H_v, NC, d->d_k, d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32,
                                  d->decay == GDR_DECAY_CHANNEL).total();
    return ok();
}

int gdr_chunk_fwd_in_workspace_bytes(const gdr_desc *d, size_t *bytes) {
    const int rc = gdr_chunk_workspace_bytes(d, bytes);
    if (rc != GDR_OK) return rc;
    // Per-channel decay: room for the convolved and normalised q, k, v.
    if (d->decay == GDR_DECAY_CHANNEL)
        *bytes += gdr::stage_ws_layout(d->B, d->T, d->H_qk, d->H_v, d->d_k,
                                       d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32).total();
    return ok();
}


int gdr_decode_step(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g, const float *beta,
                    const void *b, const void *w, float *S, void *o, void *stream) {
    int rc = validate(d, CALL_DECODE, q, k, v, g, beta, b, w, o);
    if (rc != GDR_OK) return rc;
    if (!S) return fail(GDR_E_INVAL, "S must be non-NULL");
    rc = check_alignment(d, {q, k, v, b, w, o, S}, g, beta);
    if (rc != GDR_OK) return rc;
    if (d->B == 0) return ok();
    // At most two workgroups per (sequence, V head).
    if ((long long)d->B * d->H_v * 2 > 0x7fffffffll) return fail(GDR_E_UNSUPPORTED, "B * H_v too large for one launch");
    gdr::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.bg = b; a.wg = w; a.S = S; a.o = o;
    a.B = d->B; a.Hqk = d->H_qk; a.Hv = d->H_v; a.decay = d->decay; a.scale = d->scale;
    hipError_t e = gdr::launch_decode(d->io_dtype == GDR_BF16 ? gdr::IO_BF16 : gdr::IO_F32, d->d_k, a,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}


int gdr_recurrent_fwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const void *b, const void *w, const float *S0, void *o, float *ST,
                      void *stream) {
    return recurrent_call(d, nullptr, q, k, v, g, beta, b, w, S0, o, ST, stream);
}

int gdr_chunk_fwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const void *b, const void *w, const float *S0, void *o, float *ST, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return chunk_call(d, nullptr, q, k, v, g, beta, b, w, S0, o, ST, workspace, workspace_bytes, stream);
}

int gdr_chunk_fwd_noalloc(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const void *b, const void *w, const float *S0, void *o, float *ST,
                          void *stream) {
    return chunk_call(d, nullptr, q, k, v, g, beta, b, w, S0, o, ST, nullptr, 0, stream, true);
}

int gdr_chunk_fwd_in(const gdr_desc *d, const gdr_input_stage *stage, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, const void *b, const void *w, const float *S0, void *o,
                     float *ST, void *workspace, size_t workspace_bytes, void *stream) {
    if (!stage) return fail(GDR_E_INVAL, "stage is NULL");
    return chunk_call(d, stage, q, k, v, g, beta, b, w, S0, o, ST, workspace, workspace_bytes, stream);
}

int gdr_recurrent_fwd_in(const gdr_desc *d, const gdr_input_stage *stage, const void *q, const void *k,
                         const void *v, const float *g, const float *beta, const void *b, const void *w,
                         const float *S0, void *o, float *ST, void *stream) {
    if (!stage) return fail(GDR_E_INVAL, "stage is NULL");
    return recurrent_call(d, stage, q, k, v, g, beta, b, w, S0, o, ST, stream);
}

int gdr_recurrent_bwd_workspace_bytes(const gdr_desc *d, size_t *bytes) { return bwd_workspace_bytes(d, bytes, false); }

int gdr_norm_la_workspace_bytes(const gdr_desc *d, size_t *bytes) {
    if (!bytes) return fail(GDR_E_INVAL, "bytes is NULL");
    *bytes = 0;
    if (!d) return fail(GDR_E_INVAL, "desc is NULL");
    if (d->B < 0 || d->T < 0 || d->H_v <= 0) return fail(GDR_E_INVAL, "B, T must be >= 0 and H_v > 0");
    if (d->d_k != d->d_v || !supported_dim(d->d_k))
        return fail(GDR_E_UNSUPPORTED, "d_k = %d, d_v = %d: supported are d_k == d_v in {32, 64, 128}", d->d_k, d->d_v);
    if (!size_ok(d->B, d->T, d->H_v, d->d_k)) return fail(GDR_E_INVAL, "sizes too large");
    *bytes = gdr::nla_ws_bytes(d->B, d->H_v, d->d_k, (d->T + gdr::kChunk - 1) / gdr::kChunk);
    return ok();
}

int gdr_norm_la_fwd(const gdr_desc *d, const void *phq, const void *phk, const void *v, const float *S0,
                    const float *z0, void *o, float *ST, float *zT, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return nla_call(d, false, phq, phk, v, S0, z0, o, ST, zT, workspace, workspace_bytes, stream);
}

int gdr_norm_la_decode_step(const gdr_desc *d, const void *phq, const void *phk, const void *v, float *S, float *z,
                            void *o, void *stream) {
    return nla_call(d, true, phq, phk, v, S, z, o, S, z, nullptr, 0, stream);
}

int gdr_recurrent_bwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const void *b, const void *w, const float *S0, const void *dO,
                      const float *dST, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *db,
                      float *dw, float *dS0, void *workspace, size_t workspace_bytes, void *stream) {
    return bwd_call(false, d, q, k, v, g, beta, b, w, S0, dO, dST, dq, dk, dv, dg, dbeta, db, dw, dS0, workspace,
                    workspace_bytes, stream);
}

int gdr_chunk_bwd_workspace_bytes(const gdr_desc *d, size_t *bytes) { return bwd_workspace_bytes(d, bytes, true); }

int gdr_chunk_bwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const void *b, const void *w, const float *S0, const void *dO, const float *dST, float *dq,
                  float *dk, float *dv, float *dg, float *dbeta, float *db, float *dw, float *dS0, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return bwd_call(true, d, q, k, v, g, beta, b, w, S0, dO, dST, dq, dk, dv, dg, dbeta, db, dw, dS0, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"
