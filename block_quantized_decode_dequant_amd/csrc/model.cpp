// model.cpp -- the decode step: sequencing of the per-token kernels, HIP
// graph capture and replay, and the host-streamed layer mode.
//
// The ntransformer write-up's engine ("Architecture": inference/engine over
// model/ attention, FFN and normalization) runs one Llama block per layer
// ("Main features") and keeps some layers resident in GPU memory while the
// others are copied from pinned host RAM, double buffered so the copy of the
// next layer overlaps the compute of the current one ("Performance": 3-tier
// cache; "Main features": streaming that overlaps transfer and compute).
//
// Every step is enqueued on the caller's stream.  Token and position live in
// device memory, so one captured HIP graph replays unchanged for every
// token; the argmax kernel writes the next token and advances the position.
//
// The third tier ("Performance": 3-tier cache with an NVMe/mmap fallback;
// "NVMe direct streaming": disk -> pinned staging -> host-to-device copy ->
// GPU buffer -> compute) serves the last layers from a file.  A reader
// thread reads blob j into one of two pinned staging buffers; only after that
// read has finished does the host enqueue the copy of blob j and the compute
// of its layer, so no GPU work ever waits on host progress: a failed read
// ends the step with NT_EIO and leaves nothing queued that could wait
// forever.
#include <fcntl.h>
#include <linux/aio_abi.h>
#include <sys/stat.h>
#include <sys/syscall.h>
#include <unistd.h>

#include <hip/hip_runtime.h>

#include <cerrno>
#include <chrono>
#include <cstdlib>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "nt_internal.h"

namespace nt {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t x, n, q, k, v, o, g, u, attn, pick, total;
};

nt_attn_desc attn_of(const nt_model_config &c) {
    nt_attn_desc a;
    a.n_q_heads = c.n_q_heads;
    a.n_kv_heads = c.n_kv_heads;
    a.head_dim = c.head_dim;
    a.ctx_cap = c.ctx_cap;
    a.scale = 0.f;
    a.rope_theta = c.rope_theta;     // the attention kernel rotates q and k itself
    return a;
}

Layout layout_of(const nt_model_config &c) {
    Layout L{};
    const size_t H = size_t(c.hidden), QD = size_t(c.n_q_heads) * c.head_dim,
                 KD = size_t(c.n_kv_heads) * c.head_dim, F = size_t(c.ffn);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t at = off; off += align_up(bytes); return at; };
    L.x = take(4 * H);
    L.n = take(4 * H);
    L.q = take(4 * QD);
    L.k = take(4 * KD);
    L.v = take(4 * KD);
    L.o = take(4 * QD);
    L.g = take(4 * F);
    L.u = take(4 * F);
    L.attn = take(attn_workspace_bytes(attn_of(c)));
    L.pick = take(16);                 // the greedy pick's atomic key and ticket
    L.total = off;
    return L;
}

bool config_ok(const nt_model_config &c, std::string &why) {
    if (c.n_layers < 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 ||
        c.ffn <= 0 || c.vocab <= 0 || c.ctx_cap <= 0) {
        why = "sizes must be positive";
        return false;
    }
    if (!attn_shape_ok(attn_of(c))) {
        why = "need head_dim 64 or 128 and n_q_heads / n_kv_heads in {1, 2, 4, 8}";
        return false;
    }
    if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f)) {
        why = "need rms_eps >= 0 and rope_theta > 0";
        return false;
    }
    return true;
}

bool tensor_ok(const nt_tensor_ref &t, int64_t cols, bool allow_null, std::string &why, const char *name) {
    const nt_qtype q = nt_qtype(t.type);
    if (!is_quant(q)) {
        why = std::string(name) + ": unsupported weight type";
        return false;
    }
    if (cols % block_elems(q) != 0 || cols > kMaxGemvCols) {
        why = std::string(name) + ": column count is not a whole number of blocks (or above 65536)";
        return false;
    }
    if (!t.data) {
        if (allow_null) return true;
        why = std::string(name) + ": null data";
        return false;
    }
    if (!aligned(t.data, 16)) {
        why = std::string(name) + ": data not 16-byte aligned";
        return false;
    }
    return true;
}

const int kBlobOrder = 7;   // wq, wk, wv, wo, w_gate, w_up, w_down

size_t matrix_bytes(const nt_model_config &c, int which, nt_qtype t) {
    const int64_t H = c.hidden, QD = int64_t(c.n_q_heads) * c.head_dim, KD = int64_t(c.n_kv_heads) * c.head_dim,
                  F = c.ffn;
    int64_t rows = 0, cols = 0;
    switch (which) {
    case 0: rows = QD; cols = H; break;
    case 1: case 2: rows = KD; cols = H; break;
    case 3: rows = H; cols = QD; break;
    case 4: case 5: rows = F; cols = H; break;
    default: rows = H; cols = F; break;
    }
    return size_t(rows) * size_t(cols / block_elems(t) * block_bytes(t));
}

constexpr uint64_t kFileAlign = 4096;     // O_DIRECT buffer, offset and length granule

double host_seconds() {
    return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

// O_DIRECT reads go through two library-owned bounce chunks: the kernel
// cannot hand HIP-pinned host memory to a direct block read (the read fails
// with EFAULT), so each chunk lands in ordinary aligned memory and is copied
// into the pinned staging buffer while the next chunk is read (Linux native
// asynchronous I/O; a plain blocking read when it is not available).
constexpr size_t kChunk = size_t(32) << 20;

long sys_io_setup(unsigned n, aio_context_t *ctx) { return syscall(SYS_io_setup, n, ctx); }
long sys_io_destroy(aio_context_t ctx) { return syscall(SYS_io_destroy, ctx); }
long sys_io_submit(aio_context_t ctx, long n, struct iocb **v) { return syscall(SYS_io_submit, ctx, n, v); }
long sys_io_getevents(aio_context_t ctx, long lo, long hi, struct io_event *ev, struct timespec *to) {
    return syscall(SYS_io_getevents, ctx, lo, hi, ev, to);
}

}  // namespace

// The file tier: blob j of the file layers sits at offset + j * stride.  One
// reader thread serves read requests (blob j into staging slot j % 2) in
// order; before it overwrites a slot it waits for the host-to-device copy
// out of that slot that was enqueued last.
struct FileTier {
    int fd = -1;
    bool direct = false;
    int device = 0;
    int32_t first = 0, count = 0;         // file layers [first, first + count)
    uint64_t offset = 0, stride = 0;
    size_t blob = 0, read_len = 0;        // blob bytes, bytes read per blob (blob rounded up to kFileAlign)
    void *staging[2] = {nullptr, nullptr};
    hipEvent_t staged_free[2] = {nullptr, nullptr};   // recorded after each copy out of a slot
    void *bounce[2] = {nullptr, nullptr};             // O_DIRECT only: kChunk bytes each, 4096-aligned
    aio_context_t aio = 0;                            // O_DIRECT only, when native AIO is available

    std::thread th;
    std::mutex mu;
    std::condition_variable cv;
    struct Job { int f; int slot; bool wait_copy; };
    std::deque<Job> queue;
    int outstanding = 0;                  // posted, not yet finished
    bool quit = false;
    // per step, per file layer: 0 not done, 1 read, 2 failed
    std::vector<int> state;
    std::vector<std::string> err;
    std::vector<double> t0, t1;
    uint64_t reads = 0, read_bytes = 0;

    void run() {
        (void)hipSetDevice(device);
        for (;;) {
            Job j{};
            {
                std::unique_lock<std::mutex> lk(mu);
                cv.wait(lk, [&] { return quit || !queue.empty(); });
                if (queue.empty()) return;      // quit with nothing left
                j = queue.front();
                queue.pop_front();
            }
            std::string e;
            const double a = host_seconds();
            if (j.wait_copy) {
                const hipError_t he = hipEventSynchronize(staged_free[j.slot]);
                if (he != hipSuccess) {
                    e = std::string("waiting for the staging buffer: ") + hipGetErrorString(he);
                    (void)hipGetLastError();
                }
            }
            size_t got = 0;
            if (e.empty()) {
                uint8_t *dst = static_cast<uint8_t *>(staging[j.slot]);
                const uint64_t off = offset + uint64_t(j.f) * stride;
                got = direct ? (aio ? read_aio(dst, off, e) : read_bounced(dst, off, e)) : read_plain(dst, off, e);
                if (e.empty() && got < blob)
                    e = "the file ends inside blob " + std::to_string(j.f) + " (" + std::to_string(got) + " of " +
                        std::to_string(blob) + " bytes)";
            }
            const double z = host_seconds();
            {
                std::lock_guard<std::mutex> lk(mu);
                state[j.f] = e.empty() ? 1 : 2;
                err[j.f] = e;
                t0[j.f] = a;
                t1[j.f] = z;
                if (e.empty()) {
                    ++reads;
                    read_bytes += blob;
                }
                --outstanding;
            }
            cv.notify_all();
        }
    }
    // blocking reads straight into the destination (through the page cache)
    size_t read_plain(uint8_t *dst, uint64_t off, std::string &e) {
        size_t got = 0;
        while (got < read_len) {
            const ssize_t r = pread(fd, dst + got, read_len - got, off_t(off + got));
            if (r < 0) {
                if (errno == EINTR) continue;
                e = std::string("read failed: ") + std::strerror(errno);
                break;
            }
            if (r == 0) break;              // end of file
            got += size_t(r);
        }
        return got;
    }
    // O_DIRECT, blocking, one chunk at a time through bounce[0]
    size_t read_bounced(uint8_t *dst, uint64_t off, std::string &e) {
        size_t got = 0;
        while (got < read_len) {
            const size_t want = std::min(kChunk, read_len - got);
            ssize_t r;
            do {
                r = pread(fd, bounce[0], want, off_t(off + got));
            } while (r < 0 && errno == EINTR);
            if (r < 0) {
                e = std::string("read failed: ") + std::strerror(errno);
                break;
            }
            std::memcpy(dst + got, bounce[0], size_t(r));
            got += size_t(r);
            if (size_t(r) < want) break;    // end of file
        }
        return got;
    }
    // O_DIRECT with native AIO: chunk c + 1 is read into one bounce chunk
    // while chunk c is copied out of the other
    size_t read_aio(uint8_t *dst, uint64_t off, std::string &e) {
        const size_t nch = (read_len + kChunk - 1) / kChunk;
        struct iocb cb[2];
        auto submit = [&](size_t c) -> bool {
            struct iocb &x = cb[c & 1];
            std::memset(&x, 0, sizeof(x));
            x.aio_lio_opcode = IOCB_CMD_PREAD;
            x.aio_fildes = uint32_t(fd);
            x.aio_buf = uint64_t(uintptr_t(bounce[c & 1]));
            x.aio_nbytes = std::min(kChunk, read_len - c * kChunk);
            x.aio_offset = int64_t(off + c * kChunk);
            x.aio_data = c;
            struct iocb *v[1] = {&x};
            long r;
            do {
                r = sys_io_submit(aio, 1, v);
            } while (r < 0 && errno == EINTR);
            if (r != 1) e = std::string("read submission failed: ") + std::strerror(errno);
            return r == 1;
        };
        // waits for the one read in flight; its byte count, or -1 on error
        auto complete = [&]() -> long {
            struct io_event ev;
            struct timespec to = {60, 0};
            long r;
            do {
                r = sys_io_getevents(aio, 1, 1, &ev, &to);
            } while (r < 0 && errno == EINTR);
            if (r != 1) {
                e = r == 0 ? "read timed out after 60 s" : std::string("read wait failed: ") + std::strerror(errno);
                return -1;
            }
            if (ev.res < 0) {
                e = std::string("read failed: ") + std::strerror(int(-ev.res));
                return -1;
            }
            return long(ev.res);
        };
        size_t got = 0;
        if (!submit(0)) return 0;
        for (size_t c = 0; c < nch; ++c) {
            const long r = complete();
            if (r < 0) return got;          // nothing else is in flight
            const size_t want = std::min(kChunk, read_len - c * kChunk);
            const bool more = size_t(r) == want && c + 1 < nch;
            if (more && !submit(c + 1)) return got;
            std::memcpy(dst + c * kChunk, bounce[c & 1], size_t(r));
            got += size_t(r);
            if (!more) {
                if (size_t(r) < want) break;    // end of file: nothing was submitted after it
            }
        }
        return got;
    }
    void post(int f, int slot, bool wait_copy) {
        {
            std::lock_guard<std::mutex> lk(mu);
            queue.push_back({f, slot, wait_copy});
            ++outstanding;
        }
        cv.notify_all();
    }
    // blocks until blob f is read; false (with the reason) if the read failed
    bool wait(int f, std::string &why) {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return state[f] != 0; });
        if (state[f] == 2) {
            why = err[f];
            return false;
        }
        return true;
    }
    // drops queued requests and waits for the one in progress
    void drain() {
        std::unique_lock<std::mutex> lk(mu);
        outstanding -= int(queue.size());
        queue.clear();
        cv.wait(lk, [&] { return outstanding == 0; });
    }
    void begin_step() {
        std::lock_guard<std::mutex> lk(mu);
        state.assign(size_t(count), 0);
        err.assign(size_t(count), std::string());
        t0.assign(size_t(count), 0.0);
        t1.assign(size_t(count), 0.0);
    }
    ~FileTier() {
        if (th.joinable()) {
            drain();
            {
                std::lock_guard<std::mutex> lk(mu);
                quit = true;
            }
            cv.notify_all();
            th.join();
        }
        for (int b = 0; b < 2; ++b) {
            if (staged_free[b]) (void)hipEventDestroy(staged_free[b]);
            std::free(bounce[b]);
        }
        if (aio) (void)sys_io_destroy(aio);
        if (fd >= 0) close(fd);
    }
};

}  // namespace nt

using namespace nt;

struct nt_model {
    nt_model_config cfg{};
    nt_model_weights w{};
    std::vector<nt_layer_weights> layers;
    nt_attn_desc attn{};
    Layout lay{};
    uint8_t *ws = nullptr;

    bool graph_enabled = true;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    const void *cap_args[4] = {nullptr, nullptr, nullptr, nullptr};
    hipStream_t cap_stream = nullptr;

    // host-streamed layers
    bool streaming = false;
    int32_t first_streamed = 0;
    std::vector<const void *> blobs;
    void *d_buf[2] = {nullptr, nullptr};
    size_t blob_bytes = 0, blob_off[kBlobOrder] = {};
    int32_t blob_types[kBlobOrder] = {};
    hipStream_t copy_stream = nullptr;
    hipEvent_t ready[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
    std::vector<hipEvent_t> copy_t0, copy_t1, comp_t0, comp_t1;
    hipEvent_t step_t0 = nullptr, step_t1 = nullptr;
    bool have_step = false;
    uint64_t steps = 0, layers_streamed = 0, h2d_bytes = 0;
    // the file tier (layers [file->first, n_layers)), when enabled
    std::unique_ptr<FileTier> file;
    bool staged_used[2] = {false, false};

    float *f(size_t off) const { return reinterpret_cast<float *>(ws + off); }
    void drop_graph() {
        if (exec) (void)hipGraphExecDestroy(exec);
        if (graph) (void)hipGraphDestroy(graph);
        exec = nullptr;
        graph = nullptr;
    }
    void drop_events() {
        auto kill = [](hipEvent_t &e) { if (e) (void)hipEventDestroy(e); e = nullptr; };
        for (int b = 0; b < 2; ++b) { kill(ready[b]); kill(freed[b]); }
        for (auto *v : {&copy_t0, &copy_t1, &comp_t0, &comp_t1}) {
            for (auto &e : *v) kill(e);
            v->clear();
        }
        kill(step_t0);
        kill(step_t1);
        file.reset();
        staged_used[0] = staged_used[1] = false;
    }
};

namespace nt {
namespace {

#define NT_TRY(expr)                          \
    do {                                      \
        hipError_t e_ = (expr);               \
        if (e_ != hipSuccess) return e_;      \
    } while (0)

// ys[i] = W_i . RMSNorm(x, gain) for cnt <= 3 matrices of width cols.  Runs
// of one format whose shape the LDS-ring kernels take go out as one launch
// that normalizes x itself; any other matrix reads a normalized copy in nbuf,
// made once.
hipError_t norm_gemvs(int cnt, const nt_tensor_ref *mats, const int64_t *rows, float *const *ys, int64_t cols,
                      const float *x, const float *gain, float eps, float *nbuf, hipStream_t st) {
    // exactly two runs of one format each (q/k in one format, v in another):
    // one paired launch when both take the shared layout
    int split = 1;
    while (split < cnt && mats[split].type == mats[0].type) ++split;
    bool two_runs = split < cnt && split <= 3 && cnt - split <= 3;
    for (int s = split; two_runs && s < cnt; ++s) two_runs = mats[s].type == mats[split].type;
    for (int s = 0; two_runs && s < cnt; ++s) two_runs = gemv_pair_ok(nt_qtype(mats[s].type), rows[s], cols);
    if (two_runs) {
        const void *Wa[3] = {nullptr, nullptr, nullptr}, *Wb[3] = {nullptr, nullptr, nullptr};
        for (int s = 0; s < split; ++s) Wa[s] = mats[s].data;
        for (int s = split; s < cnt; ++s) Wb[s - split] = mats[s].data;
        return launch_gemv_pair(nt_qtype(mats[0].type), split, Wa, rows, ys, nt_qtype(mats[split].type), cnt - split,
                                Wb, rows + split, ys + split, cols, x, gain, eps, st);
    }
    bool have_n = false;
    for (int i = 0; i < cnt;) {
        const nt_qtype t = nt_qtype(mats[i].type);
        if (gemv_fast_ok(t, rows[i], cols)) {
            int j = i + 1;
            while (j < cnt && mats[j].type == mats[i].type && gemv_fast_ok(t, rows[j], cols)) ++j;
            const void *W[3] = {nullptr, nullptr, nullptr};
            for (int s = i; s < j; ++s) W[s - i] = mats[s].data;
            NT_TRY(launch_gemv_multi(t, j - i, W, rows + i, ys + i, cols, x, gain, eps, 0, st));
            i = j;
        } else {
            if (!have_n) NT_TRY(launch_rmsnorm(x, gain, nbuf, cols, eps, st));
            have_n = true;
            NT_TRY(launch_gemv(t, mats[i].data, nbuf, ys[i], rows[i], cols, 0, st));
            ++i;
        }
    }
    return hipSuccess;
}

// One transformer block.  mats[i] follow the blob order.
hipError_t run_layer(nt_model *m, int l, const nt_tensor_ref *mats, const float *attn_norm, const float *ffn_norm,
                     const int32_t *d_pos, hipStream_t st) {
    const nt_model_config &c = m->cfg;
    const int64_t H = c.hidden, QD = int64_t(c.n_q_heads) * c.head_dim, KD = int64_t(c.n_kv_heads) * c.head_dim;
    float *x = m->f(m->lay.x), *n = m->f(m->lay.n), *q = m->f(m->lay.q), *k = m->f(m->lay.k);
    float *v = m->f(m->lay.v), *o = m->f(m->lay.o), *g = m->f(m->lay.g), *u = m->f(m->lay.u);
    const size_t layer_kv = size_t(c.n_kv_heads) * c.ctx_cap * c.head_dim;
    uint16_t *kc = m->w.k_cache + l * layer_kv, *vc = m->w.v_cache + l * layer_kv;

    // attention: q, k, v from the normalized residual; RoPE, cache append and
    // attend in the attention kernels
    const int64_t qkv_rows[3] = {QD, KD, KD};
    float *const qkv_out[3] = {q, k, v};
    NT_TRY(norm_gemvs(3, mats, qkv_rows, qkv_out, H, x, attn_norm, c.rms_eps, n, st));
    NT_TRY(launch_attn(m->attn, q, k, v, kc, vc, d_pos, o, m->ws + m->lay.attn, st));
    NT_TRY(launch_gemv(nt_qtype(mats[3].type), mats[3].data, o, x, H, QD, 1, st));

    // feed-forward: silu(gate) * up from the normalized residual, then down
    const nt_qtype tg = nt_qtype(mats[4].type);
    if (mats[4].type == mats[5].type && gemv_fast_ok(tg, c.ffn, H)) {
        NT_TRY(launch_gemv_swiglu(tg, mats[4].data, mats[5].data, c.ffn, H, x, ffn_norm, c.rms_eps, g, st));
    } else {
        const int64_t ff_rows[2] = {c.ffn, c.ffn};
        float *const ff_out[2] = {g, u};
        NT_TRY(norm_gemvs(2, mats + 4, ff_rows, ff_out, H, x, ffn_norm, c.rms_eps, n, st));
        NT_TRY(launch_swiglu(g, u, g, c.ffn, st));
    }
    NT_TRY(launch_gemv(nt_qtype(mats[6].type), mats[6].data, g, x, H, c.ffn, 1, st));
    return hipSuccess;
}

void resident_mats(const nt_layer_weights &L, nt_tensor_ref *mats) {
    mats[0] = L.wq; mats[1] = L.wk; mats[2] = L.wv; mats[3] = L.wo;
    mats[4] = L.w_gate; mats[5] = L.w_up; mats[6] = L.w_down;
}

hipError_t head(nt_model *m, int32_t *d_pos, float *logits, int32_t *d_next, hipStream_t st) {
    const nt_model_config &c = m->cfg;
    float *x = m->f(m->lay.x), *n = m->f(m->lay.n);
    const int64_t rows[1] = {c.vocab};
    float *const out[1] = {logits};
    NT_TRY(norm_gemvs(1, &m->w.output, rows, out, c.hidden, x, m->w.output_norm, c.rms_eps, n, st));
    NT_TRY(launch_argmax_multi(logits, c.vocab, m->ws + m->lay.pick, d_next, d_pos, st));
    return hipSuccess;
}

hipError_t enqueue_resident(nt_model *m, const int32_t *d_token, int32_t *d_pos, float *logits, int32_t *d_next,
                            hipStream_t st) {
    const nt_model_config &c = m->cfg;
    NT_TRY(launch_embed(nt_qtype(m->w.tok_embd.type), m->w.tok_embd.data, c.vocab, c.hidden, d_token,
                        m->f(m->lay.x), st));
    nt_tensor_ref mats[kBlobOrder];
    for (int l = 0; l < c.n_layers; ++l) {
        resident_mats(m->layers[l], mats);
        NT_TRY(run_layer(m, l, mats, m->layers[l].attn_norm, m->layers[l].ffn_norm, d_pos, st));
    }
    return head(m, d_pos, logits, d_next, st);
}

hipError_t prefetch(nt_model *m, int s) {
    const int b = s & 1;
    NT_TRY(hipStreamWaitEvent(m->copy_stream, m->freed[b], 0));
    NT_TRY(hipEventRecord(m->copy_t0[s], m->copy_stream));
    NT_TRY(hipMemcpyAsync(m->d_buf[b], m->blobs[s], m->blob_bytes, hipMemcpyHostToDevice, m->copy_stream));
    NT_TRY(hipEventRecord(m->copy_t1[s], m->copy_stream));
    NT_TRY(hipEventRecord(m->ready[b], m->copy_stream));
    return hipSuccess;
}

// A streamed step: layers [first_streamed, first_file) come from pinned host
// blobs copied ahead on the copy stream; layers from first_file on come from
// the file, each copied only once its read has finished.  d_buf[s % 2] holds
// streamed layer s.  On a failed read the step stops enqueuing (nothing
// queued waits on work that is not queued) and returns the read's message
// in `why`.
hipError_t enqueue_streamed(nt_model *m, const int32_t *d_token, int32_t *d_pos, float *logits, int32_t *d_next,
                            hipStream_t st, std::string &why) {
    const nt_model_config &c = m->cfg;
    const int ns = c.n_layers - m->first_streamed;
    FileTier *ft = m->file.get();
    const int nf = ft ? ft->count : 0, np = ns - nf;
    NT_TRY(hipEventRecord(m->step_t0, st));
    // file reads start at once: they depend on nothing the step computes
    if (nf > 0) {
        ft->drain();                     // nothing is left over from a step that stopped early
        ft->begin_step();
        for (int f = 0; f < 2 && f < nf; ++f) ft->post(f, f, m->staged_used[f]);
    }
    // the copy side stream must not run ahead of work already queued on the
    // compute stream that still reads the staging buffers
    if (np > 0) NT_TRY(prefetch(m, 0));
    if (np > 1) NT_TRY(prefetch(m, 1));
    NT_TRY(launch_embed(nt_qtype(m->w.tok_embd.type), m->w.tok_embd.data, c.vocab, c.hidden, d_token,
                        m->f(m->lay.x), st));
    nt_tensor_ref mats[kBlobOrder];
    for (int l = 0; l < m->first_streamed; ++l) {
        resident_mats(m->layers[l], mats);
        NT_TRY(run_layer(m, l, mats, m->layers[l].attn_norm, m->layers[l].ffn_norm, d_pos, st));
    }
    for (int s = 0; s < ns; ++s) {
        const int l = m->first_streamed + s, b = s & 1;
        if (s >= np) {
            // file layer f: wait (on the host) for its read, then copy it
            const int f = s - np, slot = f & 1;
            if (!ft->wait(f, why)) {
                ft->drain();
                return hipErrorFileNotFound;      // reported as NT_EIO with `why`
            }
            NT_TRY(hipStreamWaitEvent(m->copy_stream, m->freed[b], 0));
            NT_TRY(hipEventRecord(m->copy_t0[s], m->copy_stream));
            NT_TRY(hipMemcpyAsync(m->d_buf[b], ft->staging[slot], m->blob_bytes, hipMemcpyHostToDevice,
                                  m->copy_stream));
            NT_TRY(hipEventRecord(m->copy_t1[s], m->copy_stream));
            NT_TRY(hipEventRecord(m->ready[b], m->copy_stream));
            NT_TRY(hipEventRecord(ft->staged_free[slot], m->copy_stream));
            m->staged_used[slot] = true;
            if (f + 2 < nf) ft->post(f + 2, slot, true);
        }
        NT_TRY(hipStreamWaitEvent(st, m->ready[b], 0));
        NT_TRY(hipEventRecord(m->comp_t0[s], st));
        for (int i = 0; i < kBlobOrder; ++i) {
            mats[i].type = m->blob_types[i];
            mats[i].data = static_cast<const uint8_t *>(m->d_buf[b]) + m->blob_off[i];
        }
        NT_TRY(run_layer(m, l, mats, m->layers[l].attn_norm, m->layers[l].ffn_norm, d_pos, st));
        NT_TRY(hipEventRecord(m->comp_t1[s], st));
        NT_TRY(hipEventRecord(m->freed[b], st));
        if (s + 2 < np) NT_TRY(prefetch(m, s + 2));
    }
    NT_TRY(head(m, d_pos, logits, d_next, st));
    NT_TRY(hipEventRecord(m->step_t1, st));
    m->have_step = true;
    m->steps += 1;
    m->layers_streamed += uint64_t(ns);
    m->h2d_bytes += uint64_t(ns) * m->blob_bytes;
    return hipSuccess;
}

nt_status hip_fail(hipError_t e, const char *what) {
    (void)hipGetLastError();
    return fail(NT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

nt_status device_present() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return fail(NT_ENODEV, "no HIP device available");
    }
    return NT_OK;
}

}  // namespace
}  // namespace nt

extern "C" {

size_t nt_model_workspace_bytes(const nt_model_config *cfg) {
    std::string why;
    if (!cfg || !config_ok(*cfg, why)) return 0;
    return layout_of(*cfg).total;
}

nt_status nt_layer_blob_layout(const nt_model_config *cfg, const int32_t types[7], size_t offsets[7],
                               size_t *blob_bytes) {
    set_error("");
    std::string why;
    if (!cfg || !types || !offsets || !blob_bytes) return fail(NT_EINVAL, "nt_layer_blob_layout: null pointer");
    if (!config_ok(*cfg, why)) return fail(NT_ESHAPE, "nt_layer_blob_layout: " + why);
    size_t off = 0;
    for (int i = 0; i < kBlobOrder; ++i) {
        const nt_qtype t = nt_qtype(types[i]);
        if (!is_quant(t)) return fail(NT_EINVAL, "nt_layer_blob_layout: unsupported type");
        const int64_t cols = (i == 3) ? int64_t(cfg->n_q_heads) * cfg->head_dim : (i == 6) ? cfg->ffn : cfg->hidden;
        if (cols % block_elems(t) != 0) return fail(NT_ESHAPE, "nt_layer_blob_layout: columns not a whole number of blocks");
        offsets[i] = off;
        off += align_up(matrix_bytes(*cfg, i, t));
    }
    *blob_bytes = off;
    return NT_OK;
}

nt_status nt_model_create(const nt_model_config *cfg, const nt_model_weights *w, nt_model **out) {
    set_error("");
    if (!cfg || !w || !out) return fail(NT_EINVAL, "nt_model_create: null pointer");
    *out = nullptr;
    std::string why;
    if (!config_ok(*cfg, why)) return fail(NT_ESHAPE, "nt_model_create: " + why);
    const int64_t H = cfg->hidden, QD = int64_t(cfg->n_q_heads) * cfg->head_dim, F = cfg->ffn;
    if (!tensor_ok(w->tok_embd, H, false, why, "tok_embd") || !tensor_ok(w->output, H, false, why, "output"))
        return fail(NT_ESHAPE, "nt_model_create: " + why);
    if (!w->output_norm || !w->k_cache || !w->v_cache || !w->workspace || (cfg->n_layers > 0 && !w->layers))
        return fail(NT_EINVAL, "nt_model_create: null pointer");
    if (!aligned(w->k_cache, 16) || !aligned(w->v_cache, 16) || !aligned(w->workspace, kAlign) ||
        !aligned(w->output_norm, 4))
        return fail(NT_EALIGN, "nt_model_create: misaligned cache, workspace or gain");
    const Layout lay = layout_of(*cfg);
    if (w->workspace_bytes < lay.total) return fail(NT_ENOMEM, "nt_model_create: workspace too small");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const nt_layer_weights &L = w->layers[l];
        const nt_tensor_ref *mats[kBlobOrder] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.w_gate, &L.w_up, &L.w_down};
        const int64_t cols[kBlobOrder] = {H, H, H, QD, H, H, F};
        const char *names[kBlobOrder] = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"};
        for (int i = 0; i < kBlobOrder; ++i)
            if (!tensor_ok(*mats[i], cols[i], true, why, names[i]))
                return fail(NT_ESHAPE, "nt_model_create: layer " + std::to_string(l) + " " + why);
        if (!L.attn_norm || !L.ffn_norm) return fail(NT_EINVAL, "nt_model_create: null norm gain");
    }
    if (nt_status s = device_present()) return s;
    nt_model *m = new nt_model();
    m->cfg = *cfg;
    m->w = *w;
    m->layers.assign(w->layers, w->layers + cfg->n_layers);
    m->w.layers = nullptr;
    m->attn = attn_of(*cfg);
    m->lay = lay;
    m->ws = static_cast<uint8_t *>(w->workspace);
    // the greedy pick's key and ticket start at zero (each pick leaves them so)
    if (hipMemset(m->ws + lay.pick, 0, 16) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        delete m;
        return fail(NT_EHIP, "nt_model_create: clearing the workspace failed");
    }
    *out = m;
    return NT_OK;
}

void nt_model_destroy(nt_model *m) {
    if (!m) return;
    m->drop_graph();
    m->drop_events();
    delete m;
}

nt_status nt_model_set_graph(nt_model *m, int enable) {
    set_error("");
    if (!m) return fail(NT_EINVAL, "nt_model_set_graph: null model");
    m->graph_enabled = enable != 0;
    if (!m->graph_enabled) m->drop_graph();
    return NT_OK;
}

nt_status nt_decode_step(nt_model *m, const int32_t *d_token, int32_t *d_pos, float *logits, int32_t *d_next,
                         nt_stream stream) {
    set_error("");
    if (!m || !d_token || !d_pos || !logits || !d_next) return fail(NT_EINVAL, "nt_decode_step: null pointer");
    if (!aligned(d_token, 4) || !aligned(d_pos, 4) || !aligned(d_next, 4) || !aligned(logits, 4))
        return fail(NT_EALIGN, "nt_decode_step: misaligned pointer");
    hipStream_t st = as_stream(stream);
    if (m->streaming) {
        std::string why;
        hipError_t e = enqueue_streamed(m, d_token, d_pos, logits, d_next, st, why);
        if (!why.empty()) return fail(NT_EIO, "nt_decode_step: file tier: " + why);
        return e == hipSuccess ? NT_OK : hip_fail(e, "nt_decode_step (streamed)");
    }
    for (int l = 0; l < m->cfg.n_layers; ++l) {
        const nt_layer_weights &L = m->layers[l];
        if (!L.wq.data || !L.wk.data || !L.wv.data || !L.wo.data || !L.w_gate.data || !L.w_up.data || !L.w_down.data)
            return fail(NT_ESTATE, "nt_decode_step: layer " + std::to_string(l) +
                                       " has no resident weights and streaming is off");
    }
    if (!m->graph_enabled || st == nullptr) {
        hipError_t e = enqueue_resident(m, d_token, d_pos, logits, d_next, st);
        return e == hipSuccess ? NT_OK : hip_fail(e, "nt_decode_step");
    }
    const void *args[4] = {d_token, d_pos, logits, d_next};
    if (!m->exec || m->cap_stream != st || std::memcmp(args, m->cap_args, sizeof(args)) != 0) {
        m->drop_graph();
        hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) return hip_fail(e, "nt_decode_step: begin capture");
        hipError_t e2 = enqueue_resident(m, d_token, d_pos, logits, d_next, st);
        hipGraph_t g = nullptr;
        e = hipStreamEndCapture(st, &g);
        if (e2 != hipSuccess || e != hipSuccess) {
            if (g) (void)hipGraphDestroy(g);
            return hip_fail(e2 != hipSuccess ? e2 : e, "nt_decode_step: capture");
        }
        m->graph = g;
        e = hipGraphInstantiate(&m->exec, g, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            m->drop_graph();
            return hip_fail(e, "nt_decode_step: instantiate");
        }
        std::memcpy(m->cap_args, args, sizeof(args));
        m->cap_stream = st;
    }
    hipError_t e = hipGraphLaunch(m->exec, st);
    return e == hipSuccess ? NT_OK : hip_fail(e, "nt_decode_step: graph launch");
}

nt_status nt_stream_layers_tiered(nt_model *m, const nt_stream_desc *d, const nt_file_tier *file) {
    set_error("");
    if (!m) return fail(NT_EINVAL, "nt_stream_layers: null model");
    if (!d) {
        if (file) return fail(NT_EINVAL, "nt_stream_layers: a file tier needs a stream descriptor");
        if (m->streaming) (void)hipStreamSynchronize(m->copy_stream);
        m->streaming = false;
        m->drop_events();
        return NT_OK;
    }
    const nt_model_config &c = m->cfg;
    if (d->first_streamed_layer < 0 || d->first_streamed_layer > c.n_layers)
        return fail(NT_EINVAL, "nt_stream_layers: first_streamed_layer out of range");
    const int ns = c.n_layers - d->first_streamed_layer;
    const int first_file = file ? file->first_file_layer : c.n_layers;
    if (first_file < d->first_streamed_layer || first_file > c.n_layers)
        return fail(NT_EINVAL, "nt_stream_layers: first_file_layer must lie in [first_streamed_layer, n_layers]");
    const int nf = c.n_layers - first_file, np = ns - nf;
    if (ns > 0 && (!d->d_buf[0] || !d->d_buf[1] || !d->copy_stream))
        return fail(NT_EINVAL, "nt_stream_layers: null pointer");
    if (np > 0 && !d->h_layer_blobs) return fail(NT_EINVAL, "nt_stream_layers: null blob array");
    for (int l = 0; l < d->first_streamed_layer; ++l) {
        const nt_layer_weights &L = m->layers[l];
        if (!L.wq.data || !L.wk.data || !L.wv.data || !L.wo.data || !L.w_gate.data || !L.w_up.data || !L.w_down.data)
            return fail(NT_ESTATE, "nt_stream_layers: resident layer " + std::to_string(l) + " has no weights");
    }
    int32_t types[kBlobOrder] = {};
    size_t offs[kBlobOrder] = {}, bytes = 0;
    if (ns > 0) {
        const nt_layer_weights &F0 = m->layers[d->first_streamed_layer];
        const nt_tensor_ref *mats0[kBlobOrder] = {&F0.wq, &F0.wk, &F0.wv, &F0.wo, &F0.w_gate, &F0.w_up, &F0.w_down};
        for (int i = 0; i < kBlobOrder; ++i) types[i] = mats0[i]->type;
        for (int s = 1; s < ns; ++s) {
            const nt_layer_weights &L = m->layers[d->first_streamed_layer + s];
            const nt_tensor_ref *mats[kBlobOrder] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.w_gate, &L.w_up, &L.w_down};
            for (int i = 0; i < kBlobOrder; ++i)
                if (mats[i]->type != types[i])
                    return fail(NT_ESHAPE, "nt_stream_layers: streamed layers must share matrix types");
        }
        if (nt_status s = nt_layer_blob_layout(&c, types, offs, &bytes)) return s;
        if (d->buf_bytes < bytes) return fail(NT_ENOMEM, "nt_stream_layers: staging buffers smaller than a blob");
        if (!aligned(d->d_buf[0], kAlign) || !aligned(d->d_buf[1], kAlign))
            return fail(NT_EALIGN, "nt_stream_layers: staging buffers must be 256-byte aligned");
        for (int s = 0; s < np; ++s) {
            const void *h = d->h_layer_blobs[s];
            if (!h) return fail(NT_EINVAL, "nt_stream_layers: null blob");
            hipPointerAttribute_t attr;
            if (hipPointerGetAttributes(&attr, h) != hipSuccess || attr.type != hipMemoryTypeHost) {
                (void)hipGetLastError();
                return fail(NT_ESTATE, "nt_stream_layers: blob " + std::to_string(s) + " is not pinned host memory");
            }
        }
    }
    // the file tier: checked and opened before any state changes
    std::unique_ptr<FileTier> ft;
    if (nf > 0) {
        const uint64_t read_len = (uint64_t(bytes) + kFileAlign - 1) / kFileAlign * kFileAlign;
        if (!file->path) return fail(NT_EINVAL, "nt_stream_layers: null file path");
        if (file->offset % kFileAlign || file->stride % kFileAlign)
            return fail(NT_EALIGN, "nt_stream_layers: file offset and stride must be multiples of 4096");
        if (file->stride < bytes) return fail(NT_EINVAL, "nt_stream_layers: file stride smaller than a blob");
        if (file->staging_bytes < read_len)
            return fail(NT_ENOMEM, "nt_stream_layers: file staging buffers smaller than a blob rounded up to 4096");
        for (int b = 0; b < 2; ++b) {
            const void *h = file->h_staging[b];
            if (!h) return fail(NT_EINVAL, "nt_stream_layers: null file staging buffer");
            if (!aligned(h, kFileAlign)) return fail(NT_EALIGN, "nt_stream_layers: file staging buffers must be 4096-byte aligned");
            hipPointerAttribute_t attr;
            if (hipPointerGetAttributes(&attr, h) != hipSuccess || attr.type != hipMemoryTypeHost) {
                (void)hipGetLastError();
                return fail(NT_ESTATE, "nt_stream_layers: file staging buffer " + std::to_string(b) +
                                           " is not pinned host memory");
            }
        }
        ft.reset(new FileTier());
        int fd = -1;
        if (file->direct) {
            fd = open(file->path, O_RDONLY | O_DIRECT | O_CLOEXEC);
            ft->direct = fd >= 0;
        }
        if (fd < 0) fd = open(file->path, O_RDONLY | O_CLOEXEC);   // the file system refused O_DIRECT, or not asked
        if (fd < 0) return fail(NT_EIO, std::string("nt_stream_layers: cannot open the layer file: ") + std::strerror(errno));
        ft->fd = fd;
        struct stat sb;
        if (fstat(fd, &sb) != 0) return fail(NT_EIO, "nt_stream_layers: cannot stat the layer file");
        const uint64_t need = file->offset + uint64_t(nf - 1) * file->stride + bytes;
        if (uint64_t(sb.st_size) < need)
            return fail(NT_EINVAL, "nt_stream_layers: the layer file is shorter than its " + std::to_string(nf) +
                                       " blobs (" + std::to_string(sb.st_size) + " < " + std::to_string(need) + ")");
        if (ft->direct) {
            for (int b = 0; b < 2; ++b)
                if (posix_memalign(&ft->bounce[b], kFileAlign, kChunk) != 0) {
                    ft->bounce[b] = nullptr;
                    return fail(NT_ENOMEM, "nt_stream_layers: cannot allocate the host bounce buffers for O_DIRECT reads");
                }
            aio_context_t ctx = 0;
            if (sys_io_setup(4, &ctx) == 0) ft->aio = ctx;   // else blocking O_DIRECT reads
        }
        ft->first = first_file;
        ft->count = nf;
        ft->offset = file->offset;
        ft->stride = file->stride;
        ft->blob = bytes;
        ft->read_len = size_t(read_len);
        ft->staging[0] = file->h_staging[0];
        ft->staging[1] = file->h_staging[1];
    }
    if (nt_status s = device_present()) return s;
    if (m->streaming) (void)hipStreamSynchronize(m->copy_stream);
    m->drop_events();
    m->drop_graph();
    auto mk = [](hipEvent_t *e) { return hipEventCreate(e); };
    hipError_t e = hipSuccess;
    for (int b = 0; b < 2 && e == hipSuccess; ++b) {
        e = mk(&m->ready[b]);
        if (e == hipSuccess) e = mk(&m->freed[b]);
        if (e == hipSuccess && ft) e = hipEventCreateWithFlags(&ft->staged_free[b], hipEventDisableTiming);
    }
    m->copy_t0.assign(size_t(ns), nullptr);
    m->copy_t1.assign(size_t(ns), nullptr);
    m->comp_t0.assign(size_t(ns), nullptr);
    m->comp_t1.assign(size_t(ns), nullptr);
    for (int s = 0; s < ns && e == hipSuccess; ++s) {
        e = mk(&m->copy_t0[s]);
        if (e == hipSuccess) e = mk(&m->copy_t1[s]);
        if (e == hipSuccess) e = mk(&m->comp_t0[s]);
        if (e == hipSuccess) e = mk(&m->comp_t1[s]);
    }
    if (e == hipSuccess) e = mk(&m->step_t0);
    if (e == hipSuccess) e = mk(&m->step_t1);
    if (e == hipSuccess && ft) e = hipGetDevice(&ft->device);
    if (e != hipSuccess) {
        m->drop_events();
        return hip_fail(e, "nt_stream_layers: event creation");
    }
    if (ft) {
        ft->begin_step();
        FileTier *raw = ft.get();
        try {
            ft->th = std::thread([raw] { raw->run(); });
        } catch (...) {
            m->drop_events();
            return fail(NT_ESTATE, "nt_stream_layers: cannot start the file reader thread");
        }
        m->file = std::move(ft);
    }
    m->first_streamed = d->first_streamed_layer;
    m->blobs.assign(d->h_layer_blobs ? d->h_layer_blobs : nullptr,
                    d->h_layer_blobs ? d->h_layer_blobs + np : nullptr);
    m->d_buf[0] = d->d_buf[0];
    m->d_buf[1] = d->d_buf[1];
    m->blob_bytes = bytes;
    std::memcpy(m->blob_off, offs, sizeof(offs));
    std::memcpy(m->blob_types, types, sizeof(types));
    m->copy_stream = as_stream(d->copy_stream);
    m->streaming = true;
    m->have_step = false;
    m->steps = m->layers_streamed = m->h2d_bytes = 0;
    return NT_OK;
}

nt_status nt_stream_layers(nt_model *m, const nt_stream_desc *d) { return nt_stream_layers_tiered(m, d, nullptr); }

nt_status nt_tier_plan(const nt_model_config *cfg, const int32_t types[7], uint64_t vram_bytes,
                       uint64_t pinned_bytes, int32_t *first_streamed, int32_t *first_file) {
    set_error("");
    if (!cfg || !types || !first_streamed || !first_file) return fail(NT_EINVAL, "nt_tier_plan: null pointer");
    size_t offs[kBlobOrder], bytes = 0;
    if (nt_status s = nt_layer_blob_layout(cfg, types, offs, &bytes)) return s;
    const uint64_t L = uint64_t(cfg->n_layers);
    const uint64_t in_vram = std::min<uint64_t>(L, vram_bytes / bytes);
    const uint64_t in_ram = std::min<uint64_t>(L - in_vram, pinned_bytes / bytes);
    *first_streamed = int32_t(in_vram);
    *first_file = int32_t(in_vram + in_ram);
    return NT_OK;
}

nt_status nt_stream_stats_get(nt_model *m, nt_stream_stats *out) {
    set_error("");
    if (!m || !out) return fail(NT_EINVAL, "nt_stream_stats_get: null pointer");
    std::memset(out, 0, sizeof(*out));
    if (!m->streaming) return fail(NT_ESTATE, "nt_stream_stats_get: streaming is off");
    out->steps = m->steps;
    out->layers_streamed = m->layers_streamed;
    out->h2d_bytes = m->h2d_bytes;
    if (!m->have_step) return NT_OK;
    hipError_t e = hipEventSynchronize(m->step_t1);
    if (e != hipSuccess) return hip_fail(e, "nt_stream_stats_get");
    float ms = 0.f;
    double copy = 0.0, comp = 0.0;
    for (size_t s = 0; s < m->copy_t0.size(); ++s) {
        if (hipEventElapsedTime(&ms, m->copy_t0[s], m->copy_t1[s]) == hipSuccess) copy += ms;
        if (hipEventElapsedTime(&ms, m->comp_t0[s], m->comp_t1[s]) == hipSuccess) comp += ms;
    }
    (void)hipGetLastError();
    out->copy_ms = copy;
    out->compute_ms = comp;
    if (hipEventElapsedTime(&ms, m->step_t0, m->step_t1) == hipSuccess) out->wall_ms = ms;
    (void)hipGetLastError();
    return NT_OK;
}

nt_status nt_file_stats_get(nt_model *m, nt_file_stats *out) {
    set_error("");
    if (!m || !out) return fail(NT_EINVAL, "nt_file_stats_get: null pointer");
    std::memset(out, 0, sizeof(*out));
    FileTier *ft = m->file.get();
    if (!m->streaming || !ft) return fail(NT_ESTATE, "nt_file_stats_get: no file tier");
    std::lock_guard<std::mutex> lk(ft->mu);
    out->reads = ft->reads;
    out->read_bytes = ft->read_bytes;
    out->direct = ft->direct ? 1 : 0;
    out->file_layers = ft->count;
    double busy = 0.0, lo = 0.0, hi = 0.0;
    bool any = false;
    for (int f = 0; f < ft->count; ++f) {
        if (ft->state[f] != 1) continue;
        busy += ft->t1[f] - ft->t0[f];
        if (!any || ft->t0[f] < lo) lo = ft->t0[f];
        if (!any || ft->t1[f] > hi) hi = ft->t1[f];
        any = true;
    }
    out->read_ms = busy * 1e3;
    out->read_span_ms = any ? (hi - lo) * 1e3 : 0.0;
    return NT_OK;
}

}  // extern "C"
