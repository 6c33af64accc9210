// Decoder layers around the link step (include/piclink.h: pic_link_forward, pic_linear,
// pic_rmsnorm): the selected rows' hidden states go through every layer of a multi-layer store,
// with the link step as each layer's attention.
//
// EPIC (atlas.scime.ai summary, "Approach"): only the recomputed rows (the first k tokens of every
// chunk, and the suffix) run through the model at link time; every other token's K/V of every layer
// comes from the compile step. "Key results" and "Limitations": 7-9B Llama-class models.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "model.h"
#include "runtime.h"

namespace piclink {
namespace {

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Activation buffers of the selected rows, after the plan's workspace.
struct Activations {
    int64_t h, q, k, v, attn, act, end;
};

Activations activation_layout(const pic_store *s, const pic_plan *plan, const pic_model_config &m) {
    const int64_t R = (int64_t)plan->row_pos.size();
    const int64_t hd = s->cfg.head_dim;
    Activations a{};
    int64_t off = align256(plan->workspace_bytes);
    auto place = [&](int64_t elems) {
        const int64_t at = off;
        off = align256(off + elems * 2);
        return at;
    };
    a.h = place(R * m.d_model);
    a.q = place(R * s->cfg.num_q_heads * hd);
    a.k = place(R * s->cfg.num_kv_heads * hd);
    a.v = place(R * s->cfg.num_kv_heads * hd);
    a.attn = place(R * s->cfg.num_q_heads * hd);
    a.act = place(R * m.d_ff);
    a.end = off;
    return a;
}

void check_model(const pic_store *s, const pic_model_config *m) {
    if (!m) fail(PIC_ERR_INVALID, "null model config");
    if (s->cfg.dtype != PIC_DTYPE_BF16) fail(PIC_ERR_INVALID, "the decoder layers run on bfloat16 stores");
    const int64_t qd = (int64_t)s->cfg.num_q_heads * s->cfg.head_dim;
    const int64_t kvd = (int64_t)s->cfg.num_kv_heads * s->cfg.head_dim;
    if (m->d_model != qd) fail(PIC_ERR_INVALID, "d_model must equal num_q_heads * head_dim");
    if (m->d_model % 128 != 0) fail(PIC_ERR_INVALID, "d_model must be a multiple of 128");
    if (m->d_model > 8192) fail(PIC_ERR_INVALID, "d_model must be at most 8,192");
    if ((qd + 2 * kvd) % 128 != 0 || kvd % 64 != 0)
        fail(PIC_ERR_INVALID, "(Hq + 2 Hkv) * head_dim must be a multiple of 128 and Hkv * head_dim of 64");
    if (m->d_ff <= 0 || m->d_ff % 64 != 0) fail(PIC_ERR_INVALID, "d_ff must be a positive multiple of 64");
    if (!(m->norm_eps > 0.0f)) fail(PIC_ERR_INVALID, "norm_eps must be positive");
}

}  // namespace
}  // namespace piclink

using namespace piclink;

extern "C" {

pic_status pic_forward_workspace(const pic_store *s, const pic_plan *plan, const pic_model_config *m,
                                 int64_t *bytes) {
    return guarded([&] {
        if (!s || !plan || !bytes) fail(PIC_ERR_INVALID, "null argument");
        if (plan->owner != s) fail(PIC_ERR_INVALID, "plan belongs to another store");
        check_model(s, m);
        *bytes = activation_layout(s, plan, *m).end;
    });
}

pic_status pic_link_forward(pic_store *s, const pic_plan *plan, const pic_model_config *m,
                            const pic_layer_weights *layers, void *x, void *workspace, int64_t workspace_bytes,
                            hipStream_t stream) {
    return guarded([&] {
        if (!s || !plan || !layers) fail(PIC_ERR_INVALID, "null argument");
        if (plan->owner != s) fail(PIC_ERR_INVALID, "plan belongs to another store");
        if (!s->k_pool) fail(PIC_ERR_STATE, "metadata-only store has no device");
        check_model(s, m);
        const int L = s->cfg.num_layers;
        for (int l = 0; l < L; ++l) {
            const pic_layer_weights &w = layers[l];
            if (!w.attn_norm || !w.w_qkv || !w.w_o || !w.mlp_norm || !w.w_gate_up || !w.w_down)
                fail(PIC_ERR_INVALID, "layer " + std::to_string(l) + " has a null weight");
        }
        const Activations act = activation_layout(s, plan, *m);
        if (!workspace || workspace_bytes < act.end)
            fail(PIC_ERR_WORKSPACE, "the forward pass needs " + std::to_string(act.end) + " bytes of workspace");
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) fail(PIC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        const int R = (int)plan->row_pos.size();
        if (R == 0) return;
        if (!x) fail(PIC_ERR_INVALID, "null hidden states");
        // the plan's tables, once for every layer
        if (!s->ledger.holds(plan, workspace))
            upload_tables(s, const_cast<pic_plan *>(plan), workspace, workspace_bytes, stream);
        uint8_t *ws = static_cast<uint8_t *>(workspace);
        void *h = ws + act.h, *q = ws + act.q, *k = ws + act.k, *v = ws + act.v, *attn = ws + act.attn,
             *mlp = ws + act.act;
        const int hd = s->cfg.head_dim;
        const int qd = s->cfg.num_q_heads * hd, kvd = s->cfg.num_kv_heads * hd;
        const int dm = m->d_model, dff = m->d_ff;
        for (int l = 0; l < L; ++l) {
            const pic_layer_weights &w = layers[l];
            check_hip(launch_rmsnorm(x, w.attn_norm, h, R, dm, m->norm_eps, stream), "rmsnorm launch");
            LinearCall qkv{};
            qkv.a = h;
            qkv.w = w.w_qkv;
            qkv.m = R;
            qkv.n = qd + 2 * kvd;
            qkv.k = dm;
            qkv.epilogue = kSplit3;
            qkv.out[0] = q;
            qkv.out[1] = k;
            qkv.out[2] = v;
            qkv.ld_out[0] = qd;
            qkv.ld_out[1] = kvd;
            qkv.ld_out[2] = kvd;
            qkv.split0 = qd;
            qkv.split1 = kvd;
            check_hip(launch_linear(qkv, stream), "QKV projection launch");
            launch_link(s, plan, l, q, k, v, attn, nullptr, ws, s->profiling, stream);
            LinearCall o{};
            o.a = attn;
            o.w = w.w_o;
            o.m = R;
            o.n = dm;
            o.k = qd;
            o.epilogue = kResidual;
            o.out[0] = x;
            o.ld_out[0] = dm;
            o.residual = x;
            check_hip(launch_linear(o, stream), "output projection launch");
            check_hip(launch_rmsnorm(x, w.mlp_norm, h, R, dm, m->norm_eps, stream), "rmsnorm launch");
            LinearCall gu{};
            gu.a = h;
            gu.w = w.w_gate_up;
            gu.m = R;
            gu.n = 2 * dff;
            gu.k = dm;
            gu.epilogue = kSwiGlu;
            gu.out[0] = mlp;
            gu.ld_out[0] = dff;
            check_hip(launch_linear(gu, stream), "gate/up projection launch");
            LinearCall down{};
            down.a = mlp;
            down.w = w.w_down;
            down.m = R;
            down.n = dm;
            down.k = dff;
            down.epilogue = kResidual;
            down.out[0] = x;
            down.ld_out[0] = dm;
            down.residual = x;
            check_hip(launch_linear(down, stream), "down projection launch");
        }
    });
}

pic_status pic_linear(const void *a, const void *w, void *out, int32_t m, int32_t n, int32_t k, int32_t epilogue,
                      const void *residual, hipStream_t stream) {
    return guarded([&] {
        if (m < 0 || n <= 0 || k <= 0 || n % 128 != 0 || k % 64 != 0)
            fail(PIC_ERR_INVALID, "m >= 0, n a positive multiple of 128 and k of 64");
        if (epilogue < 0 || epilogue > 2) fail(PIC_ERR_INVALID, "epilogue must be 0, 1 or 2");
        if (m == 0) return;
        if (!a || !w || !out || (epilogue == 1 && !residual)) fail(PIC_ERR_INVALID, "null tensor");
        LinearCall c{};
        c.a = a;
        c.w = w;
        c.m = m;
        c.n = n;
        c.k = k;
        c.epilogue = epilogue;
        c.out[0] = out;
        c.ld_out[0] = epilogue == kSwiGlu ? n / 2 : n;
        c.residual = epilogue == kResidual ? residual : nullptr;
        check_hip(launch_linear(c, stream), "linear launch");
    });
}

pic_status pic_rmsnorm(const void *x, const void *w, void *y, int32_t rows, int32_t dm, float eps,
                       hipStream_t stream) {
    return guarded([&] {
        if (rows < 0 || dm <= 0 || dm % 8 != 0 || dm > 8192) fail(PIC_ERR_INVALID, "dm must be a multiple of 8 up to 8,192");
        if (!(eps > 0.0f)) fail(PIC_ERR_INVALID, "eps must be positive");
        if (rows == 0) return;
        if (!x || !w || !y) fail(PIC_ERR_INVALID, "null tensor");
        check_hip(launch_rmsnorm(x, w, y, rows, dm, eps, stream), "rmsnorm launch");
    });
}

}  // extern "C"
