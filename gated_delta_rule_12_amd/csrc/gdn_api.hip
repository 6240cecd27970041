// C ABI of libgdn: argument validation, workspace sizing, dispatch between
// the MFMA and vector-ALU kernel families, and optional per-kernel timing
// through a caller-owned timer.
#include <string.h>

#include <new>

#include <string>
#include <vector>

#include "gdn_internal.h"
#include "../../include/gdn.h"

// A caller-owned per-kernel timer: one record per distinct kernel name, the
// HIP event pairs not yet read, and a pool of spare events.  Touched only by
// the calls it is passed to.
struct gdn_timer {
    struct Ev { int kernel; hipEvent_t a, b; };
    std::vector<std::string> names;
    std::vector<Ev> events;
    std::vector<hipEvent_t> pool;
    std::vector<double> ms;
    std::vector<int64_t> cnt;
    int open = -1;
    hipEvent_t open_a = nullptr;

    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    void drain() {
        for (auto& ev : events) {
            float t = 0.f;
            if (hipEventSynchronize(ev.b) == hipSuccess && hipEventElapsedTime(&t, ev.a, ev.b) == hipSuccess) {
                ms[ev.kernel] += t;
                cnt[ev.kernel] += 1;
            }
            pool.push_back(ev.a);
            pool.push_back(ev.b);
        }
        events.clear();
    }
    ~gdn_timer() {
        drain();
        for (hipEvent_t e : pool) hipEventDestroy(e);
    }
};

namespace gdn {
namespace {

bool dim_ok(int64_t d) { return d >= 16 && d <= 128 && d % 16 == 0; }
bool chunk_ok(int32_t c) { return c == 16 || c == 32 || c == 64; }

int validate(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
             int32_t dtype, int32_t gate, int32_t order, int32_t n_segments) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_E_ARG;
    if (gate != GDN_GATE_SCALAR && gate != GDN_GATE_CHANNEL) return GDN_E_ARG;
    if (order != GDN_PREDICT_THEN_DECAY && order != GDN_DECAY_THEN_PREDICT) return GDN_E_ARG;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || chunk <= 0 || n_segments <= 0)
        return GDN_E_SHAPE;
    // grid limits: chunks and heads map onto grid dimensions
    if (H > 65535 || B > 65535 || T / chunk > (int64_t)1 << 30) return GDN_E_SHAPE;
    if (!dim_ok(dk) || !dim_ok(dv) || !chunk_ok(chunk)) return GDN_E_UNSUPPORTED;
    if (H * (int64_t)n_segments > 65535) return GDN_E_UNSUPPORTED;
    return GDN_OK;
}

Problem make_problem(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                     int32_t dtype, int32_t gate, int32_t order, float scale) {
    Problem p{};
    p.B = B; p.T = T; p.H = H; p.dk = dk; p.dv = dv;
    p.C = chunk;
    p.NC = (int)((T + chunk - 1) / chunk);
    p.dtype = dtype; p.gate = gate; p.order = order; p.scale = scale;
    return p;
}

WsLayout layout_for(const Problem& p, const Split& sp) {
    return mfma_supported(p.dk, p.dv, p.C, p.dtype, p.gate) ? mfma_layout(p, sp)
                                                             : valu_layout(p, sp);
}

int auto_segments(const Problem& p) {
    return mfma_supported(p.dk, p.dv, p.C, p.dtype, p.gate) ? mfma_auto_segments(p) : 1;
}

// the segments an explicit request of n runs in (n, or a multiple of it)
int run_segments(const Problem& p, int n) {
    return mfma_supported(p.dk, p.dv, p.C, p.dtype, p.gate) ? mfma_refine_segments(p, n) : n;
}

int finish(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_E_HIP; }

// The kernels move q, k, v, a per-channel gate, the states and the output in
// 16-byte pieces; beta and a scalar gate per float.
bool aligned(const void* ptr, uintptr_t a) { return (uintptr_t)ptr % a == 0; }
bool forward_aligned(const void* q, const void* k, const void* v, const float* alpha, int gate,
                     const float* beta, const float* state0, const float* out, const float* state_out) {
    return aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(state0, 16) &&
           aligned(out, 16) && aligned(state_out, 16) && aligned(beta, 4) &&
           aligned(alpha, gate == GDN_GATE_CHANNEL ? 16 : 4);
}

int run_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                int32_t dtype, int32_t gate, int32_t order, float scale, int32_t n_segments,
                const void* q, const void* k, const void* v, const float* alpha,
                const float* beta, const float* state0, float* out, float* state_out,
                void* workspace, size_t workspace_bytes, void* stream, gdn_timer* timer,
                bool raw = false) {
    // n_segments == 0: the library picks the schedule (gdn_chunk_fwd)
    int s = validate(B, T, H, dk, dv, chunk, dtype, gate, order, n_segments > 0 ? n_segments : 1);
    if (s != GDN_OK) return s;
    Problem p = make_problem(B, T, H, dk, dv, chunk, dtype, gate, order, scale);
    if (B * H == 0) return GDN_OK;
    n_segments = n_segments == 0 ? auto_segments(p) : run_segments(p, n_segments);
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return GDN_E_ARG;
    if (!forward_aligned(q, k, v, alpha, gate, beta, state0, out, state_out)) return GDN_E_ARG;
    p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
    p.s0 = state0; p.out = out; p.s_out = state_out;
    p.timer = timer;
    p.raw = raw ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.NC == 0) return finish(copy_state(p, st));
    const Split sp = make_split(p.NC, n_segments);
    if (raw && !mfma_supported(dk, dv, chunk, dtype, gate)) {
        // vector-ALU family: the prologue writes normalised fp32 inputs into
        // the workspace (after the forward's own part), then the fp32 forward
        Problem pf = p;
        pf.dtype = GDN_F32;
        pf.raw = 0;
        const size_t base = align256(valu_layout(pf, sp).total);
        if (!workspace || workspace_bytes < base + raw_inputs_bytes(p)) return GDN_E_WORKSPACE;
        if (!aligned(workspace, 16)) return GDN_E_ARG;
        char* ws = static_cast<char*>(workspace);
        const RawInputs r = raw_inputs_at(p, ws + base);
        const hipError_t e = raw_prologue(p, r, st);
        if (e != hipSuccess) return GDN_E_HIP;
        pf.q = r.q; pf.k = r.k; pf.v = r.v; pf.alpha = r.alpha; pf.beta = r.beta;
        return finish(valu_forward(pf, sp, ws, st));
    }
    const WsLayout L = layout_for(p, sp);
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return GDN_E_WORKSPACE;
    if (!aligned(workspace, 16)) return GDN_E_ARG;  // (moved in 16-byte pieces)
    char* ws = static_cast<char*>(workspace);
    if (mfma_supported(dk, dv, chunk, dtype, gate)) return finish(mfma_forward(p, sp, ws, st));
    return finish(valu_forward(p, sp, ws, st));
}

int decode_common(int64_t B, int64_t H, int64_t dk, int64_t dv, int32_t dtype, int32_t gate,
                  int32_t order, float scale, const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta, const float* state_in, float* out,
                  float* state_out, bool prologue, void* stream, gdn_timer* timer) {
    int s = validate(B, 1, H, dk, dv, 16, dtype, gate, order, 1);
    if (s != GDN_OK) return s;
    if (B * H == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !out || !state_out) return GDN_E_ARG;
    // the kernel moves q, k (and a vector gate) and the state rows in 16-byte
    // (fp32) or 8-byte (bf16) pieces
    const uintptr_t qk_align = dtype == GDN_BF16 ? 8 : 16;
    if (((uintptr_t)q | (uintptr_t)k) % qk_align != 0) return GDN_E_ARG;
    if (((uintptr_t)state_in | (uintptr_t)state_out) % 16 != 0) return GDN_E_ARG;
    if (gate == GDN_GATE_CHANNEL && (uintptr_t)alpha % 16 != 0) return GDN_E_ARG;
    Problem p = make_problem(B, 1, H, dk, dv, 16, dtype, gate, order, scale);
    p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
    p.s0 = state_in; p.out = out; p.s_out = state_out;
    p.timer = timer;
    return finish(decode_step(p, prologue, static_cast<hipStream_t>(stream)));
}

}  // namespace

void prof_begin(gdn_timer* t, const char* name, hipStream_t st) {
    if (!t) return;
    int idx = -1;
    for (size_t i = 0; i < t->names.size(); ++i)
        if (t->names[i] == name) idx = (int)i;
    if (idx < 0) {
        t->names.emplace_back(name);
        t->ms.push_back(0.0);
        t->cnt.push_back(0);
        idx = (int)t->names.size() - 1;
    }
    t->open = idx;
    t->open_a = t->get();
    if (t->open_a) hipEventRecord(t->open_a, st);
}

void prof_end(gdn_timer* t, hipStream_t st) {
    if (!t || t->open < 0 || !t->open_a) return;
    hipEvent_t b = t->get();
    if (b) {
        hipEventRecord(b, st);
        t->events.push_back({t->open, t->open_a, b});
    }
    t->open = -1;
    t->open_a = nullptr;
    if (t->events.size() > 4096) t->drain();
}

}  // namespace gdn

using namespace gdn;

static int backward_common(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t dtype, int32_t gate,
                 int32_t order, float scale, const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta, const float* state0, const float* grad_out,
                 const float* grad_state_out, float* grad_q, float* grad_k, float* grad_v,
                 float* grad_alpha, float* grad_beta, float* grad_state0, void* workspace,
                 size_t workspace_bytes, void* stream, gdn_timer* timer) {
    int s = validate(B, T, H, dk, dv, 16, dtype, gate, order, 1);
    if (s != GDN_OK) return s;
    if (B * H == 0) return GDN_OK;
    // one workgroup per (batch, head, block of at least 16 state rows)
    if (B * H * (dv / 16) > ((int64_t)1 << 31) - 1) return GDN_E_SHAPE;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !grad_out || !grad_q || !grad_k || !grad_v ||
                  !grad_alpha || !grad_beta))
        return GDN_E_ARG;
    // q, k move in 8-byte (bf16) or 16-byte (fp32) pieces; a channel gate, the
    // states, dq, dk, a channel dalpha and the workspace in 16-byte pieces;
    // everything else per element
    const uintptr_t qk_align = dtype == GDN_BF16 ? 8 : 16;
    const uintptr_t gate_align = gate == GDN_GATE_CHANNEL ? 16 : 4;
    if (!aligned(q, qk_align) || !aligned(k, qk_align) || !aligned(state0, 16) ||
        !aligned(grad_state_out, 16) || !aligned(grad_state0, 16) || !aligned(alpha, gate_align) ||
        !aligned(beta, 4) || !aligned(v, 2) || !aligned(grad_out, 4) || !aligned(grad_q, 16) ||
        !aligned(grad_k, 16) || !aligned(grad_v, 4) || !aligned(grad_alpha, gate_align) ||
        !aligned(grad_beta, 4) || !aligned(workspace, 16))
        return GDN_E_ARG;
    const bool chunked = chunked_backward_supported(dk, dv, gate);
    // the chunked path reads dL/d out in 16-byte pieces
    if (chunked && !aligned(grad_out, 16)) return GDN_E_ARG;
    const size_t need = chunked ? chunked_backward_workspace(B, T, H, dk) : backward_workspace(B, T, H, dk, dv, gate);
    if (T > 0 && (!workspace || workspace_bytes < need)) return GDN_E_WORKSPACE;
    BwdProblem a{};
    a.p = make_problem(B, T, H, dk, dv, 16, dtype, gate, order, scale);
    a.p.q = q; a.p.k = k; a.p.v = v; a.p.alpha = alpha; a.p.beta = beta; a.p.s0 = state0;
    a.p.timer = timer;
    a.dout = grad_out;
    a.ds_out = grad_state_out;
    a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dalpha = grad_alpha; a.dbeta = grad_beta;
    a.ds0 = grad_state0;
    if (chunked) return finish(backward_chunked(a, workspace, static_cast<hipStream_t>(stream)));
    a.ckpt = static_cast<float*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + backward_ckpt_bytes(B, T, H, dk, dv, gate));
    return finish(backward(a, static_cast<hipStream_t>(stream)));
}



extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_E_ARG: return "GDN_E_ARG: null pointer or invalid enum";
        case GDN_E_SHAPE: return "GDN_E_SHAPE: negative or inconsistent size";
        case GDN_E_UNSUPPORTED: return "GDN_E_UNSUPPORTED: dk/dv must be multiples of 16 up to 128, chunk 16, 32 or 64";
        case GDN_E_WORKSPACE: return "GDN_E_WORKSPACE: workspace missing or smaller than gdn_workspace_bytes()";
        case GDN_E_HIP: return "GDN_E_HIP: a HIP runtime call or kernel launch failed";
        case GDN_E_SCRATCH: return "GDN_E_SCRATCH: the problem needs more workspace than gdn_chunk_fwd_noalloc's static scratch (GDN_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown gdn status";
    }
}

int gdn_validate(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                 int32_t dtype, int32_t gate, int32_t order, int32_t n_segments) {
    return validate(B, T, H, dk, dv, chunk, dtype, gate, order, n_segments);
}

int gdn_chunk_path(int64_t dk, int64_t dv, int32_t chunk, int32_t dtype, int32_t gate) {
    int s = validate(1, 0, 1, dk, dv, chunk, dtype, gate, 0, 1);
    if (s != GDN_OK) return s;
    return mfma_supported(dk, dv, chunk, dtype, gate) ? GDN_PATH_MFMA : GDN_PATH_VALU;
}

int gdn_chunk_segments(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                       int32_t dtype, int32_t gate) {
    int s = validate(B, T, H, dk, dv, chunk, dtype, gate, 0, 1);
    if (s != GDN_OK) return s;
    Problem p = make_problem(B, T, H, dk, dv, chunk, dtype, gate, 0, 1.f);
    if (p.NC == 0 || B * H == 0) return 1;
    return make_split(p.NC, auto_segments(p)).G;
}

int gdn_seqpar_segments(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                        int32_t dtype, int32_t gate, int32_t n_segments) {
    int s = validate(B, T, H, dk, dv, chunk, dtype, gate, 0, n_segments);
    if (s != GDN_OK) return s;
    Problem p = make_problem(B, T, H, dk, dv, chunk, dtype, gate, 0, 1.f);
    if (p.NC == 0 || B * H == 0) return 1;
    return make_split(p.NC, run_segments(p, n_segments)).G;
}

size_t gdn_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           int32_t chunk, int32_t dtype, int32_t gate, int32_t n_segments) {
    if (validate(B, T, H, dk, dv, chunk, dtype, gate, 0, n_segments) != GDN_OK) return 0;
    Problem p = make_problem(B, T, H, dk, dv, chunk, dtype, gate, 0, 1.f);
    if (p.NC == 0 || B * H == 0) return 0;
    size_t bytes = layout_for(p, make_split(p.NC, run_segments(p, n_segments))).total;
    if (n_segments == 1) {
        // also covers gdn_chunk_fwd, whose schedule may cut sequences into segments
        const size_t a = layout_for(p, make_split(p.NC, auto_segments(p))).total;
        if (a > bytes) bytes = a;
    }
    return bytes;
}

int gdn_chunk_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                  int32_t dtype, int32_t gate, int32_t order, float scale,
                  const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta, const float* state0, float* out, float* state_out,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return run_chunked(B, T, H, dk, dv, chunk, dtype, gate, order, scale, 0, q, k, v, alpha,
                       beta, state0, out, state_out, workspace, workspace_bytes, stream, nullptr);
}

int gdn_chunk_fwd_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                        int32_t dtype, int32_t gate, int32_t order, float scale,
                        const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const float* state0, float* out, float* state_out,
                        void* workspace, size_t workspace_bytes, void* stream, gdn_timer* timer) {
    return run_chunked(B, T, H, dk, dv, chunk, dtype, gate, order, scale, 0, q, k, v, alpha,
                       beta, state0, out, state_out, workspace, workspace_bytes, stream, timer);
}

int gdn_chunk_fwd_raw(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                      int32_t dtype, int32_t gate, int32_t order, float scale,
                      const void* q, const void* k, const void* v, const float* alpha_logit,
                      const float* beta_logit, const float* state0, float* out, float* state_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return run_chunked(B, T, H, dk, dv, chunk, dtype, gate, order, scale, 0, q, k, v, alpha_logit,
                       beta_logit, state0, out, state_out, workspace, workspace_bytes, stream, nullptr,
                       true);
}

int gdn_chunk_fwd_raw_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                            int32_t dtype, int32_t gate, int32_t order, float scale,
                            const void* q, const void* k, const void* v, const float* alpha_logit,
                            const float* beta_logit, const float* state0, float* out, float* state_out,
                            void* workspace, size_t workspace_bytes, void* stream, gdn_timer* timer) {
    return run_chunked(B, T, H, dk, dv, chunk, dtype, gate, order, scale, 0, q, k, v, alpha_logit,
                       beta_logit, state0, out, state_out, workspace, workspace_bytes, stream, timer,
                       true);
}

size_t gdn_raw_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                               int32_t chunk, int32_t dtype, int32_t gate) {
    if (validate(B, T, H, dk, dv, chunk, dtype, gate, 0, 1) != GDN_OK) return 0;
    if (mfma_supported(dk, dv, chunk, dtype, gate))
        return gdn_workspace_bytes(B, T, H, dk, dv, chunk, dtype, gate, 1);
    Problem p = make_problem(B, T, H, dk, dv, chunk, GDN_F32, gate, 0, 1.f);
    if (p.NC == 0 || B * H == 0) return 0;
    return align256(valu_layout(p, make_split(p.NC, 1)).total) + raw_inputs_bytes(p);
}

int gdn_seqpar_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                   int32_t dtype, int32_t gate, int32_t order, float scale, int32_t n_segments,
                   const void* q, const void* k, const void* v, const float* alpha,
                   const float* beta, const float* state0, float* out, float* state_out,
                   void* workspace, size_t workspace_bytes, void* stream) {
    if (n_segments < 1) return GDN_E_SHAPE;  // (0 would select the library's schedule)
    return run_chunked(B, T, H, dk, dv, chunk, dtype, gate, order, scale, n_segments, q, k, v,
                       alpha, beta, state0, out, state_out, workspace, workspace_bytes, stream,
                       nullptr);
}

int gdn_seqpar_fwd_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t chunk,
                         int32_t dtype, int32_t gate, int32_t order, float scale, int32_t n_segments,
                         const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const float* state0, float* out, float* state_out,
                         void* workspace, size_t workspace_bytes, void* stream, gdn_timer* timer) {
    if (n_segments < 1) return GDN_E_SHAPE;
    return run_chunked(B, T, H, dk, dv, chunk, dtype, gate, order, scale, n_segments, q, k, v,
                       alpha, beta, state0, out, state_out, workspace, workspace_bytes, stream,
                       timer);
}

int gdn_recurrent_ref(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t dtype,
                      int32_t gate, int32_t order, float scale, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta,
                      const float* state0, float* out, float* state_out, void* stream) {
    int s = validate(B, T, H, dk, dv, 16, dtype, gate, order, 1);
    if (s != GDN_OK) return s;
    if (B * H == 0) return GDN_OK;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return GDN_E_ARG;
    if (!forward_aligned(q, k, v, alpha, gate, beta, state0, out, state_out)) return GDN_E_ARG;
    Problem p = make_problem(B, T, H, dk, dv, 16, dtype, gate, order, scale);
    p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
    p.s0 = state0; p.out = out; p.s_out = state_out;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) return finish(copy_state(p, st));
    return finish(recurrent_forward(p, st));
}

int gdn_decode_step(int64_t B, int64_t H, int64_t dk, int64_t dv, int32_t dtype, int32_t gate,
                    int32_t order, float scale, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, const float* state_in,
                    float* out, float* state_out, void* stream) {
    return decode_common(B, H, dk, dv, dtype, gate, order, scale, q, k, v, alpha, beta,
                         state_in, out, state_out, false, stream, nullptr);
}

int gdn_decode_step_timed(int64_t B, int64_t H, int64_t dk, int64_t dv, int32_t dtype, int32_t gate,
                          int32_t order, float scale, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const float* state_in,
                          float* out, float* state_out, void* stream, gdn_timer* timer) {
    return decode_common(B, H, dk, dv, dtype, gate, order, scale, q, k, v, alpha, beta,
                         state_in, out, state_out, false, stream, timer);
}

int gdn_decode_step_raw(int64_t B, int64_t H, int64_t dk, int64_t dv, int32_t dtype, int32_t gate,
                        int32_t order, float scale, const void* q, const void* k, const void* v,
                        const float* alpha_logit, const float* beta_logit, const float* state_in,
                        float* out, float* state_out, void* stream) {
    return decode_common(B, H, dk, dv, dtype, gate, order, scale, q, k, v, alpha_logit,
                         beta_logit, state_in, out, state_out, true, stream, nullptr);
}

size_t gdn_backward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    int32_t gate) {
    if (validate(B, T, H, dk, dv, 16, GDN_F32, gate, GDN_PREDICT_THEN_DECAY, 1) != GDN_OK) return 0;
    if (chunked_backward_supported(dk, dv, gate)) return chunked_backward_workspace(B, T, H, dk);
    return backward_workspace(B, T, H, dk, dv, gate);
}

int gdn_backward_path(int64_t dk, int64_t dv, int32_t gate) {
    if (validate(1, 1, 1, dk, dv, 16, GDN_F32, gate, GDN_PREDICT_THEN_DECAY, 1) != GDN_OK)
        return validate(1, 1, 1, dk, dv, 16, GDN_F32, gate, GDN_PREDICT_THEN_DECAY, 1);
    return chunked_backward_supported(dk, dv, gate) ? GDN_BWD_CHUNKED : GDN_BWD_TOKEN;
}

int gdn_backward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t dtype, int32_t gate,
                 int32_t order, float scale, const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta, const float* state0, const float* grad_out,
                 const float* grad_state_out, float* grad_q, float* grad_k, float* grad_v,
                 float* grad_alpha, float* grad_beta, float* grad_state0, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return backward_common(B, T, H, dk, dv, dtype, gate, order, scale, q, k, v, alpha, beta, state0,
                           grad_out, grad_state_out, grad_q, grad_k, grad_v, grad_alpha, grad_beta,
                           grad_state0, workspace, workspace_bytes, stream, nullptr);
}

int gdn_backward_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int32_t dtype,
                       int32_t gate, int32_t order, float scale, const void* q, const void* k,
                       const void* v, const float* alpha, const float* beta, const float* state0,
                       const float* grad_out, const float* grad_state_out, float* grad_q,
                       float* grad_k, float* grad_v, float* grad_alpha, float* grad_beta,
                       float* grad_state0, void* workspace, size_t workspace_bytes, void* stream,
                       gdn_timer* timer) {
    return backward_common(B, T, H, dk, dv, dtype, gate, order, scale, q, k, v, alpha, beta, state0,
                           grad_out, grad_state_out, grad_q, grad_k, grad_v, grad_alpha, grad_beta,
                           grad_state0, workspace, workspace_bytes, stream, timer);
}

int gdn_timer_create(gdn_timer** timer) {
    if (!timer) return GDN_E_ARG;
    *timer = new (std::nothrow) gdn_timer();
    return *timer ? GDN_OK : GDN_E_HIP;
}

int gdn_timer_destroy(gdn_timer* timer) {
    delete timer;
    return GDN_OK;
}

int gdn_timer_read(gdn_timer* timer, int index, char* name, size_t name_len, double* total_ms,
                   int64_t* count) {
    if (!timer) return GDN_E_ARG;
    timer->drain();
    if (index < 0 || index >= (int)timer->names.size()) return GDN_E_ARG;
    if (name && name_len > 0) {
        strncpy(name, timer->names[index].c_str(), name_len - 1);
        name[name_len - 1] = '\0';
    }
    if (total_ms) *total_ms = timer->ms[index];
    if (count) *count = timer->cnt[index];
    return GDN_OK;
}

}  // extern "C"
