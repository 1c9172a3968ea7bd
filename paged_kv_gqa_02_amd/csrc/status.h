// status.h -- error recording shared by the library's source files.
#pragma once

#include <hip/hip_runtime.h>

#include "paged_attn.h"

// Records `what` as this thread's paged_attn_last_error() message; returns st.
pa_status pa_record_error(pa_status st, const char* what);

// Records "where: <HIP error string>"; returns PA_ERR_HIP.
pa_status pa_record_hip_error(hipError_t e, const char* where);
