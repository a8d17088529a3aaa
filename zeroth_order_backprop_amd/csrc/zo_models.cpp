// Dispatch of forward-only loss evaluation to the model families.
#include "zo_models.hpp"

#include "zo_internal.hpp"

namespace zo {

zo_status model_check_shape(const zo_model_desc& d)
{
    switch (d.kind) {
        case ZO_MODEL_LSQ: return lsq_check(d);
        case ZO_MODEL_MLP: return mlp_check(d);
        case ZO_MODEL_DECODER: return decoder_check(d);
    }
    return fail(ZO_ERR_INVALID, "unknown model kind");
}

zo_status model_check_batch(const zo_model_desc& d, const zo_batch& b)
{
    (void)d;
    (void)b;
    return ZO_OK;
}

size_t model_workspace_bytes(const zo_model_desc& d)
{
    switch (d.kind) {
        case ZO_MODEL_LSQ: return lsq_workspace(d);
        case ZO_MODEL_MLP: return mlp_workspace(d);
        case ZO_MODEL_DECODER: return decoder_workspace(d);
    }
    return 0;
}

zo_status model_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n_perts, double* loss,
                        hipStream_t s)
{
    switch (m.desc.kind) {
        case ZO_MODEL_LSQ: return lsq_forward(m, b, perts, n_perts, loss, s);
        case ZO_MODEL_MLP: return mlp_forward(m, b, perts, n_perts, loss, s);
        case ZO_MODEL_DECODER: return decoder_forward(m, b, perts, n_perts, loss, s);
    }
    return fail(ZO_ERR_INVALID, "unknown model kind");
}

}  // namespace zo
