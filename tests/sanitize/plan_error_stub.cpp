// Host-only test builds of libwt's plan logic (plan.cpp, schedule.cpp,
// host_api.cpp) have no runtime.cpp and so no plan objects: this supplies the
// one runtime.cpp function host_api.cpp refers to. Test infrastructure only.
#include "plan.h"

namespace wt {
const char *plan_error_text(const wt_plan *) { return ""; }
}  // namespace wt
