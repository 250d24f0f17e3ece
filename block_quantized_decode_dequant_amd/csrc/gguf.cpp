// gguf.cpp -- reads the GGUF container the engine loads its models from
// (the ntransformer write-up, "Overview": GGUF models, Q4_0 / Q8_0 / Q4_K_M /
// Q5_K / Q6_K / F16 / F32).  The pages name the container but give no
// layout; this follows the public GGUF v3 definition:
//
//   u32 magic "GGUF" | u32 version (2 or 3) | u64 n_tensors | u64 n_kv
//   n_kv x   { string key | u32 value type | value }
//   n_tensors x { string name | u32 n_dims | u64 ne[n_dims] | u32 type | u64 offset }
//   padding to `general.alignment` (default 32) | tensor data
//
// strings are u64 length + bytes; value types 0..12 are u8, i8, u16, i16, u32,
// i32, f32, bool, string, array (u32 element type, u64 count, elements), u64,
// i64, f64; ne[0] is the fastest-varying dimension (a row of a weight
// matrix), and each tensor's offset counts from the start of the data area.
//
// The file is mapped read-only and every read is bounds-checked, so a
// truncated or malformed file gives an error, never a read past the mapping.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstring>
#include <string>
#include <vector>

#include "nt_internal.h"

struct nt_gguf {
    const uint8_t *base = nullptr;
    size_t size = 0;
    uint32_t version = 0;
    uint64_t alignment = 32;
    size_t data_off = 0;
    struct Kv {
        std::string key;
        uint32_t type = 0;
        uint64_t u = 0;      // unsigned / bool value
        int64_t i = 0;       // signed value
        double f = 0.0;      // floating value
        std::string s;       // string value
        uint32_t arr_type = 0;
        uint64_t arr_len = 0;
    };
    struct Tensor {
        std::string name;
        uint32_t n_dims = 0;
        uint64_t ne[4] = {1, 1, 1, 1};
        uint32_t type = 0;
        uint64_t offset = 0;
        uint64_t bytes = 0;
    };
    std::vector<Kv> kv;
    std::vector<Tensor> tensors;
};

namespace {

using nt::fail;

enum : uint32_t { U8, I8, U16, I16, U32, I32, F32V, BOOL, STR, ARR, U64, I64, F64V };

struct Reader {
    const uint8_t *p;
    size_t size, pos = 0;
    bool ok = true;
    bool need(size_t n) {
        if (!ok || n > size - pos) ok = false;
        return ok;
    }
    template <class T> T get() {
        T v{};
        if (need(sizeof(T))) {
            std::memcpy(&v, p + pos, sizeof(T));
            pos += sizeof(T);
        }
        return v;
    }
    std::string str() {
        const uint64_t n = get<uint64_t>();
        if (!ok || n > (uint64_t(1) << 32) || !need(size_t(n))) {
            ok = false;
            return {};
        }
        std::string s(reinterpret_cast<const char *>(p + pos), size_t(n));
        pos += size_t(n);
        return s;
    }
};

size_t scalar_size(uint32_t t) {
    switch (t) {
    case U8: case I8: case BOOL: return 1;
    case U16: case I16: return 2;
    case U32: case I32: case F32V: return 4;
    case U64: case I64: case F64V: return 8;
    default: return 0;
    }
}

// one scalar of type t into kv (ints to u/i, floats to f)
bool read_scalar(Reader &r, uint32_t t, nt_gguf::Kv &kv) {
    switch (t) {
    case U8: kv.u = r.get<uint8_t>(); kv.i = int64_t(kv.u); break;
    case I8: kv.i = r.get<int8_t>(); kv.u = uint64_t(kv.i); break;
    case U16: kv.u = r.get<uint16_t>(); kv.i = int64_t(kv.u); break;
    case I16: kv.i = r.get<int16_t>(); kv.u = uint64_t(kv.i); break;
    case U32: kv.u = r.get<uint32_t>(); kv.i = int64_t(kv.u); break;
    case I32: kv.i = r.get<int32_t>(); kv.u = uint64_t(kv.i); break;
    case U64: kv.u = r.get<uint64_t>(); kv.i = int64_t(kv.u); break;
    case I64: kv.i = r.get<int64_t>(); kv.u = uint64_t(kv.i); break;
    case F32V: kv.f = r.get<float>(); break;
    case F64V: kv.f = r.get<double>(); break;
    case BOOL: kv.u = r.get<uint8_t>() ? 1 : 0; kv.i = int64_t(kv.u); break;
    case STR: kv.s = r.str(); break;
    default: return false;
    }
    if (t != F32V && t != F64V) kv.f = double(t == I8 || t == I16 || t == I32 || t == I64 ? double(kv.i) : double(kv.u));
    return r.ok;
}

// bytes of a tensor of `n` elements of ggml type t, or 0 if t is unknown
uint64_t tensor_bytes(uint32_t t, uint64_t n) {
    const nt_qtype q = nt_qtype(t);
    const int64_t be = nt::block_elems(q), bb = nt::block_bytes(q);
    if (be <= 0 || bb <= 0 || n % uint64_t(be) != 0) return 0;
    return n / uint64_t(be) * uint64_t(bb);
}

nt_status parse(nt_gguf *g) {
    Reader r{g->base, g->size};
    const uint32_t magic = r.get<uint32_t>();
    if (!r.ok || magic != 0x46554747u) return fail(NT_EINVAL, "nt_gguf_open: not a GGUF file (bad magic)");
    g->version = r.get<uint32_t>();
    if (!r.ok || (g->version != 2 && g->version != 3))
        return fail(NT_EINVAL, "nt_gguf_open: unsupported GGUF version " + std::to_string(g->version));
    const uint64_t n_tensors = r.get<uint64_t>(), n_kv = r.get<uint64_t>();
    if (!r.ok || n_tensors > (uint64_t(1) << 24) || n_kv > (uint64_t(1) << 24))
        return fail(NT_EINVAL, "nt_gguf_open: truncated header or absurd counts");
    for (uint64_t k = 0; k < n_kv; ++k) {
        nt_gguf::Kv kv;
        kv.key = r.str();
        kv.type = r.get<uint32_t>();
        if (!r.ok) return fail(NT_EINVAL, "nt_gguf_open: truncated metadata");
        if (kv.type == ARR) {
            kv.arr_type = r.get<uint32_t>();
            kv.arr_len = r.get<uint64_t>();
            if (!r.ok) return fail(NT_EINVAL, "nt_gguf_open: truncated array header");
            if (kv.arr_type == STR) {
                for (uint64_t e = 0; e < kv.arr_len && r.ok; ++e) (void)r.str();
            } else {
                const size_t es = scalar_size(kv.arr_type);
                if (es == 0 || kv.arr_len > (r.size - r.pos) / es)
                    return fail(NT_EINVAL, "nt_gguf_open: bad array in key " + kv.key);
                r.pos += size_t(kv.arr_len) * es;
            }
        } else if (!read_scalar(r, kv.type, kv)) {
            return fail(NT_EINVAL, "nt_gguf_open: bad value for key " + kv.key);
        }
        if (!r.ok) return fail(NT_EINVAL, "nt_gguf_open: truncated metadata");
        if (kv.key == "general.alignment") {
            if (kv.type != U32 || kv.u == 0 || (kv.u & (kv.u - 1)) != 0)
                return fail(NT_EINVAL, "nt_gguf_open: general.alignment must be a power-of-two u32");
            g->alignment = kv.u;
        }
        g->kv.push_back(std::move(kv));
    }
    for (uint64_t k = 0; k < n_tensors; ++k) {
        nt_gguf::Tensor t;
        t.name = r.str();
        t.n_dims = r.get<uint32_t>();
        if (!r.ok || t.n_dims == 0 || t.n_dims > 4) return fail(NT_EINVAL, "nt_gguf_open: bad tensor info");
        uint64_t n = 1;
        for (uint32_t d = 0; d < t.n_dims; ++d) {
            t.ne[d] = r.get<uint64_t>();
            if (t.ne[d] == 0 || t.ne[d] > (uint64_t(1) << 40) || n > (uint64_t(1) << 40) / t.ne[d])
                return fail(NT_EINVAL, "nt_gguf_open: bad dimensions of tensor " + t.name);
            n *= t.ne[d];
        }
        t.type = r.get<uint32_t>();
        t.offset = r.get<uint64_t>();
        if (!r.ok) return fail(NT_EINVAL, "nt_gguf_open: truncated tensor info");
        t.bytes = tensor_bytes(t.type, n);
        g->tensors.push_back(std::move(t));
    }
    const uint64_t a = g->alignment;
    const uint64_t data = (uint64_t(r.pos) + a - 1) / a * a;
    if (data > g->size) return fail(NT_EINVAL, "nt_gguf_open: no data area");
    g->data_off = size_t(data);
    for (const auto &t : g->tensors) {
        if (t.offset % a != 0) return fail(NT_EINVAL, "nt_gguf_open: misaligned data of tensor " + t.name);
        if (t.bytes != 0 && (t.offset > g->size - data || t.bytes > g->size - data - t.offset))
            return fail(NT_EINVAL, "nt_gguf_open: data of tensor " + t.name + " runs past the end of the file");
    }
    return NT_OK;
}

const nt_gguf::Kv *find_kv(const nt_gguf *g, const std::string &key) {
    for (const auto &kv : g->kv)
        if (kv.key == key) return &kv;
    return nullptr;
}

}  // namespace

extern "C" {

nt_status nt_gguf_open(const char *path, nt_gguf **out) {
    nt::set_error("");
    if (!path || !out) return fail(NT_EINVAL, "nt_gguf_open: null pointer");
    *out = nullptr;
    const int fd = ::open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return fail(NT_EINVAL, std::string("nt_gguf_open: cannot open ") + path);
    struct stat st{};
    if (fstat(fd, &st) != 0 || st.st_size < 24) {
        ::close(fd);
        return fail(NT_EINVAL, std::string("nt_gguf_open: too short to be GGUF: ") + path);
    }
    void *m = mmap(nullptr, size_t(st.st_size), PROT_READ, MAP_PRIVATE, fd, 0);
    ::close(fd);
    if (m == MAP_FAILED) return fail(NT_EINVAL, std::string("nt_gguf_open: cannot map ") + path);
    nt_gguf *g = new nt_gguf();
    g->base = static_cast<const uint8_t *>(m);
    g->size = size_t(st.st_size);
    const nt_status s = parse(g);
    if (s != NT_OK) {
        nt_gguf_close(g);
        return s;
    }
    *out = g;
    return NT_OK;
}

void nt_gguf_close(nt_gguf *g) {
    if (!g) return;
    if (g->base) munmap(const_cast<uint8_t *>(g->base), g->size);
    delete g;
}

int64_t nt_gguf_tensor_count(const nt_gguf *g) { return g ? int64_t(g->tensors.size()) : -1; }

nt_status nt_gguf_tensor_info(const nt_gguf *g, int64_t i, const char **name, int32_t *type, int64_t *rows,
                              int64_t *cols, const void **data, size_t *bytes) {
    nt::set_error("");
    if (!g || !name || !type || !rows || !cols || !data || !bytes)
        return fail(NT_EINVAL, "nt_gguf_tensor_info: null pointer");
    if (i < 0 || i >= int64_t(g->tensors.size())) return fail(NT_EINVAL, "nt_gguf_tensor_info: index out of range");
    const auto &t = g->tensors[size_t(i)];
    *name = t.name.c_str();
    *type = int32_t(t.type);
    *cols = int64_t(t.ne[0]);
    *rows = int64_t(t.ne[1] * t.ne[2] * t.ne[3]);
    *bytes = size_t(t.bytes);
    *data = t.bytes ? g->base + g->data_off + t.offset : nullptr;
    if (t.bytes == 0) return fail(NT_ESHAPE, "nt_gguf_tensor_info: " + t.name + " has a type this library cannot size");
    return NT_OK;
}

int64_t nt_gguf_find_tensor(const nt_gguf *g, const char *name) {
    if (!g || !name) return -1;
    for (size_t i = 0; i < g->tensors.size(); ++i)
        if (g->tensors[i].name == name) return int64_t(i);
    return -1;
}

nt_status nt_gguf_llama_config(const nt_gguf *g, int32_t ctx_cap, nt_model_config *cfg) {
    nt::set_error("");
    if (!g || !cfg) return fail(NT_EINVAL, "nt_gguf_llama_config: null pointer");
    const auto *arch = find_kv(g, "general.architecture");
    if (!arch || arch->type != STR || arch->s != "llama")
        return fail(NT_EINVAL, "nt_gguf_llama_config: general.architecture is not \"llama\"");
    auto num = [&](const char *key, double *v) -> bool {
        const auto *kv = find_kv(g, key);
        if (!kv || kv->type == STR || kv->type == ARR) return false;
        *v = kv->f;
        return true;
    };
    double L, H, F, Hq, Hkv = -1, eps, theta = 10000.0, ctx = 0, kdim = 0, vdim = 0;
    if (!num("llama.block_count", &L) || !num("llama.embedding_length", &H) ||
        !num("llama.feed_forward_length", &F) || !num("llama.attention.head_count", &Hq) ||
        !num("llama.attention.layer_norm_rms_epsilon", &eps))
        return fail(NT_EINVAL, "nt_gguf_llama_config: a required llama.* key is missing");
    if (!num("llama.attention.head_count_kv", &Hkv)) Hkv = Hq;
    (void)num("llama.rope.freq_base", &theta);
    (void)num("llama.context_length", &ctx);
    (void)num("llama.attention.key_length", &kdim);      // head size when it is not hidden / heads
    (void)num("llama.attention.value_length", &vdim);
    const int64_t emb = nt_gguf_find_tensor(g, "token_embd.weight");
    if (emb < 0) return fail(NT_EINVAL, "nt_gguf_llama_config: no token_embd.weight");
    const auto &te = g->tensors[size_t(emb)];
    if (L < 1 || H < 1 || F < 1 || Hq < 1 || Hkv < 1 || int64_t(te.ne[0]) != int64_t(H) ||
        (kdim <= 0 && int64_t(H) % int64_t(Hq) != 0))
        return fail(NT_ESHAPE, "nt_gguf_llama_config: inconsistent llama.* sizes");
    nt_model_config c{};
    c.n_layers = int32_t(L);
    c.hidden = int32_t(H);
    c.n_q_heads = int32_t(Hq);
    c.n_kv_heads = int32_t(Hkv);
    c.head_dim = kdim > 0 ? int32_t(kdim) : int32_t(int64_t(H) / int64_t(Hq));
    c.ffn = int32_t(F);
    c.vocab = int32_t(te.ne[1]);
    c.ctx_cap = ctx_cap > 0 ? ctx_cap : int32_t(ctx);
    c.rms_eps = float(eps);
    c.rope_theta = float(theta);
    if (c.ctx_cap <= 0) return fail(NT_ESHAPE, "nt_gguf_llama_config: no context length given or stored");
    if (vdim > 0 && int32_t(vdim) != c.head_dim)   // the KV cache holds keys and values of one head size
        return fail(NT_ESHAPE, "nt_gguf_llama_config: value_length differs from the key head size");
    *cfg = c;
    return NT_OK;
}

}  // extern "C"
