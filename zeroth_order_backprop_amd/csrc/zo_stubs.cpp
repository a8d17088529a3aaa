// Model families not built yet report UNSUPPORTED.
#include "zo_internal.hpp"
#include "zo_models.hpp"

namespace zo {
zo_status decoder_check(const zo_model_desc&) { return ZO_OK; }
size_t decoder_workspace(const zo_model_desc&) { return 0; }
zo_status decoder_forward(const ModelView&, const zo_batch&, const zo_pert*, int, double*, hipStream_t)
{ return fail(ZO_ERR_UNSUPPORTED, "decoder forward not built"); }
}  // namespace zo
